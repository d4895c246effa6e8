// Weight-streaming GEMV / skinny GEMM core for gfx950.
//
// One wavefront owns a group of 16-row weight tiles and a range of k-chunks
// of the packed layout (common.hpp).  Per 32-column block it dequantises the
// tile's codes in registers into the B operand of v_mfma_f32_16x16x32_f16
// (column j = weight row, exact fp16 codes), takes the activations of up to
// 16 tokens per x-tile as the A operand, and applies the block's fp16 scale to
// the fp32 MFMA result, so every product is exact and the accumulation is
// fp32 ("Eseguire Unlimited-OCR su Apple Silicon con C e Metal", section
// "Quantizzazione": dequantisation fused into the GEMV, no fp16 copy of the
// weights).  The result layout is the MFMA D layout: lane l, register v holds
// token 16*xt + 4*(l >> 4) + v and weight row 16*tile + (l & 15).
#pragma once

#include <type_traits>

#include "common.hpp"

namespace ocrdec {

template <int FMT>
struct Geom;
template <>
struct Geom<OCRDEC_F16> { static constexpr int SB = 1, CB = 1024, SCB = 0; };
template <>
struct Geom<OCRDEC_Q8_0> { static constexpr int SB = 2, CB = 1088, SCB = 4; };
template <>
struct Geom<OCRDEC_Q4_0> { static constexpr int SB = 4, CB = 1152, SCB = 8; };
template <>
struct Geom<OCRDEC_U8A_G32> { static constexpr int SB = 2, CB = 1152, SCB = 8; };

template <int FMT>
OCR_DEV int64_t n_chunks_dev(int k) {
    constexpr int KC = 32 * Geom<FMT>::SB;
    return (k + KC - 1) / KC;
}

// Registers of one (tile, chunk) for one lane.
struct WRegs {
    uint4 q;
    uint2 s;
};

template <int FMT>
OCR_DEV void load_wchunk(const uint8_t* chunk, int lane, WRegs& r) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load((const u32x4*)(chunk + (uint32_t)lane * 16u));
    r.q = make_uint4(v.x, v.y, v.z, v.w);
    if constexpr (FMT == OCRDEC_Q4_0 || FMT == OCRDEC_U8A_G32) {
        r.s = *(const uint2*)(chunk + 1024u + ((uint32_t)lane & 15u) * 8u);
    } else if constexpr (FMT == OCRDEC_Q8_0) {
        r.s.x = *(const uint32_t*)(chunk + 1024u + ((uint32_t)lane & 15u) * 4u);
        r.s.y = 0;
    } else {
        r.s = make_uint2(0, 0);
    }
}

// load_wchunk through a buffer resource over the weights (base address in
// scalar registers) at byte offset soff of the chunk: the lane offsets are
// fixed, so a load needs no per-lane address arithmetic.
template <int FMT>
OCR_DEV void load_wchunk_rs(__amdgpu_buffer_rsrc_t rs, uint32_t soff, int lane, WRegs& r) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16, (int)soff, 2 /* nt */);
    r.q = make_uint4(v[0], v[1], v[2], v[3]);
    if constexpr (FMT == OCRDEC_Q4_0 || FMT == OCRDEC_U8A_G32) {
        const auto sv = __builtin_amdgcn_raw_buffer_load_b64(rs, 1024 + (lane & 15) * 8, (int)soff, 0);
        r.s = make_uint2(sv[0], sv[1]);
    } else if constexpr (FMT == OCRDEC_Q8_0) {
        r.s.x = __builtin_amdgcn_raw_buffer_load_b32(rs, 1024 + (lane & 15) * 4, (int)soff, 0);
        r.s.y = 0;
    } else {
        r.s = make_uint2(0, 0);
    }
}

template <int FMT>
OCR_DEV half8v wfrag(const WRegs& r, int j) {
    if constexpr (FMT == OCRDEC_F16) {
        return bits_to_half8(r.q);
    } else if constexpr (FMT == OCRDEC_Q4_0) {
        uint32_t dw = j == 0 ? r.q.x : j == 1 ? r.q.y : j == 2 ? r.q.z : r.q.w;
        return deq_q4(dw);
    } else if constexpr (FMT == OCRDEC_Q8_0) {
        return j == 0 ? deq_q8(r.q.x, r.q.y) : deq_q8(r.q.z, r.q.w);
    } else {
        return j == 0 ? deq_u8(r.q.x, r.q.y) : deq_u8(r.q.z, r.q.w);
    }
}

// fp16 scale of block j for this lane's weight row.
template <int FMT>
OCR_DEV float wscale(const WRegs& r, int j) {
    if constexpr (FMT == OCRDEC_Q4_0) {
        uint32_t w = (j < 2) ? r.s.x : r.s.y;
        return h2f((uint16_t)((j & 1) ? (w >> 16) : (w & 0xFFFF)));
    } else if constexpr (FMT == OCRDEC_Q8_0) {
        return h2f((uint16_t)(j ? (r.s.x >> 16) : (r.s.x & 0xFFFF)));
    } else if constexpr (FMT == OCRDEC_U8A_G32) {
        uint32_t w = j ? r.s.y : r.s.x;
        return h2f((uint16_t)(w & 0xFFFF));
    } else {
        return 1.0f;
    }
}

// Zero point (int8-asymmetric only).
OCR_DEV float wzero_u8a(const WRegs& r, int j) {
    uint32_t w = j ? r.s.y : r.s.x;
    return h2f((uint16_t)(w >> 16));
}

// Multiply-accumulate one (tile, chunk) into acc[XT].
// xa[j][xt]: A fragments of block j, x-tile xt; xs[j][xt]: per-token sums of
// the block's activations (int8-asymmetric only).
template <int FMT, int XT>
OCR_DEV void chunk_mac(const WRegs& w, const half8v (&xa)[Geom<FMT>::SB][XT],
                       const float4v (&xs)[Geom<FMT>::SB][XT], float4v (&acc)[XT]) {
    constexpr int SB = Geom<FMT>::SB;
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < SB; ++j) {
        half8v b = wfrag<FMT>(w, j);
        if constexpr (FMT == OCRDEC_F16) {
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) acc[xt] = mfma16(xa[j][xt], b, acc[xt]);
        } else if constexpr (FMT == OCRDEC_U8A_G32) {
            const float s = wscale<FMT>(w, j), z = wzero_u8a(w, j);
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) {
                float4v t = mfma16(xa[j][xt], b, zero);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[xt][v] = fmaf(s, fmaf(-z, xs[j][xt][v], t[v]), acc[xt][v]);
            }
        } else {
            const float d = wscale<FMT>(w, j);
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) {
                float4v t = mfma16(xa[j][xt], b, zero);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[xt][v] = fmaf(d, t[v], acc[xt][v]);
            }
        }
    }
}

// chunk_mac for the NT tiles of one chunk and one x-tile, block-scaled
// formats: every tile's block products are issued before any of them is
// scaled, so the scaling does not wait on the matrix pipe's latency.
template <int FMT, int NT>
OCR_DEV void chunk_mac_tiles(const WRegs (&w)[NT], const half8v (&xa)[Geom<FMT>::SB][1],
                             const float4v (&xs)[Geom<FMT>::SB][1], float4v (&acc)[NT][1]) {
    constexpr int SB = Geom<FMT>::SB;
    if constexpr (FMT == OCRDEC_Q4_0 || FMT == OCRDEC_Q8_0) {
        const float4v zero = {0.f, 0.f, 0.f, 0.f};
        float4v t[NT][SB];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int j = 0; j < SB; ++j) t[i][j] = mfma16(xa[j][0], wfrag<FMT>(w[i], j), zero);
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const float d = wscale<FMT>(w[i], j);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][0][v] = fmaf(d, t[i][j][v], acc[i][0][v]);
            }
    } else {
#pragma unroll
        for (int i = 0; i < NT; ++i) chunk_mac<FMT, 1>(w[i], xa, xs, acc[i]);
    }
}

// Q4_0 through raw codes (deq_q4_raw): the MFMA of block j forms
// 2^-24 sum_k x_k n_k starting from the accumulator input -2^-24 * 8 sum_k x_k,
// which leaves 2^-24 sum_k x_k q_k; the block scale is applied as for the
// other formats and the accumulators carry the factor 2^-24 until the k-loop
// ends (q4_unscale).  nb[j][xt]: that input for the chunk's block j and
// x-tile xt.  Seven VALU operations per eight weights, against eleven with
// deq_q4.
// SPLIT: the codes of deq_q4_split, for activations prepared by
// q4_split_prepare (five VALU operations per eight weights).
template <int NT, int XT, bool SPLIT = false>
OCR_DEV void chunk_mac_q4b(const WRegs* w, const half8v (&xa)[4][XT], const float4v (&nb)[4][XT],
                           float4v (&acc)[NT][XT]) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const uint32_t dw[4] = {w[i].q.x, w[i].q.y, w[i].q.z, w[i].q.w};
        float4v t[4][XT];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const half8v b = SPLIT ? deq_q4_split(dw[j]) : deq_q4_raw(dw[j]);
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) t[j][xt] = mfma16(xa[j][xt], b, nb[j][xt]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float d = wscale<OCRDEC_Q4_0>(w[i], j);
#pragma unroll
            for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[i][xt][v] = fmaf(d, t[j][xt][v], acc[i][xt][v]);
        }
    }
}

// Multiplies accumulators by s (a power of two: exact).
template <int NT, int XT>
OCR_DEV void scale_acc(float4v (&acc)[NT][XT], float s) {
#pragma unroll
    for (int i = 0; i < NT; ++i)
#pragma unroll
        for (int xt = 0; xt < XT; ++xt) acc[i][xt] *= s;
}

// -2^-24 * 8 * sum_k x[t][k] for one block's A fragment: an MFMA against the
// constant -2^-21 (an exact fp16 subnormal); every column of the result holds
// the token's sum.
OCR_DEV float4v q4_bias(const half8v& xa) {
    const uint4 c = {0x80088008u, 0x80088008u, 0x80088008u, 0x80088008u};
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    return mfma16(xa, bits_to_half8(c), zero);
}

// chunk_mac for the NT tiles of one chunk.  Q4_0 with one x-tile takes the
// raw codes, with the bias of each block formed once for all tiles (the
// accumulators then carry the factor 2^-24: the k-loop brackets its chunks
// with q4_scale / q4_unscale); the rest run chunk_mac per tile.
template <int FMT, int XT>
constexpr bool q4_raw_path() { return FMT == OCRDEC_Q4_0 && XT == 1; }
template <int FMT, int NT, int XT>
OCR_DEV void q4_scale(float4v (&acc)[NT][XT]) {
    if constexpr (q4_raw_path<FMT, XT>()) scale_acc<NT, XT>(acc, 1.0f / Q4_RAW_SCALE);
}
template <int FMT, int NT, int XT>
OCR_DEV void q4_unscale(float4v (&acc)[NT][XT]) {
    if constexpr (q4_raw_path<FMT, XT>()) scale_acc<NT, XT>(acc, Q4_RAW_SCALE);
}
template <int FMT, int NT, int XT>
OCR_DEV void chunk_mac_nt(const WRegs* w, const half8v (&xa)[Geom<FMT>::SB][XT],
                          const float4v (&xs)[Geom<FMT>::SB][XT], float4v (&acc)[NT][XT]) {
    if constexpr (q4_raw_path<FMT, XT>()) {
        // block by block (all products of a chunk at once would not fit the
        // k-loops' register budgets; with two x-tiles neither does the
        // bias, and deq_q4 serves).  The caller's loop ends with q4_unscale.
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float4v nb[XT];
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) nb[xt] = q4_bias(xa[j][xt]);
#pragma unroll
            for (int i = 0; i < NT; ++i) {
                const uint32_t dw = j == 0 ? w[i].q.x : j == 1 ? w[i].q.y : j == 2 ? w[i].q.z : w[i].q.w;
                const half8v b = deq_q4_raw(dw);
                const float d = wscale<OCRDEC_Q4_0>(w[i], j);
#pragma unroll
                for (int xt = 0; xt < XT; ++xt) {
                    const float4v t = mfma16(xa[j][xt], b, nb[xt]);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[i][xt][v] = fmaf(d, t[v], acc[i][xt][v]);
                }
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < NT; ++i) chunk_mac<FMT, XT>(w[i], xa, xs, acc[i]);
    }
}

// For chunk_mac_q4b<.., SPLIT> over LDS-staged activations, once per
// workgroup: divides positions 2, 3, 6, 7 of every 8-column group of the
// staged rows by 16 in place (exact for normal results; a value below 2^-10
// keeps its subnormal quotient's 2^-25 absolute rounding) and writes
// tab[16 j + t] = -2^-24 * 8 * sum_k x[t][k] of block j and token t over the
// values as stored (an MFMA against -2^-21 at positions 0, 1, 4, 5 and -2^-17
// at the divided ones), for blocks j < nblk_pad; blocks from nblk on and
// tokens from ntok on give 0.  Each lane rewrites exactly the piece it then
// reads; wave w takes blocks w, w + waves, ...  The caller waits for the
// workgroup afterwards.
OCR_DEV void q4_split_prepare(uint16_t* xl, int ldl, int ntok, int nblk, int nblk_pad, float* tab) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint4 cu = {0x80088008u, 0x80808080u, 0x80088008u, 0x80808080u};
    const half8v coef = bits_to_half8(cu);
    const half2v sixteenth = {(f16_t)0.0625f, (f16_t)0.0625f};
    const float4v zero = {0.f, 0.f, 0.f, 0.f};
    for (int j = wave; j < nblk_pad; j += nw) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < nblk) {
            uint4* pc = (uint4*)(xl + (lane & 15) * ldl + j * 32 + 8 * (lane >> 4));
            v = *pc;
            v.y = h2_to_u32(u32_to_h2(v.y) * sixteenth);
            v.w = h2_to_u32(u32_to_h2(v.w) * sixteenth);
            *pc = v;
            if ((lane & 15) >= ntok) v = make_uint4(0, 0, 0, 0);
        }
        const float4v u = mfma16(bits_to_half8(v), coef, zero);
        if ((lane & 15) == 0) *(float4v*)(tab + 16 * j + 4 * (lane >> 4)) = u;
    }
}

// Activation source: token i of the current x-tile set -> fp16 row pointer
// (row: NULL past the last token; rowc: clamped to the last token, rows >= 1).
struct XDirect {
    const uint16_t* x;
    int64_t ld;
    int rows;
    OCR_DEV const uint16_t* row(int tok) const { return tok < rows ? x + (int64_t)tok * ld : nullptr; }
    OCR_DEV const uint16_t* rowc(int tok) const { return x + (int64_t)min(tok, rows - 1) * ld; }
};

// Gathered activations: token i -> x[map[i]] (grouped MoE rows).
struct XGather {
    const uint16_t* x;
    int64_t ld;
    const int32_t* map;
    int rows;
    OCR_DEV const uint16_t* row(int tok) const {
        return tok < rows ? x + (int64_t)map[tok] * ld : nullptr;
    }
    OCR_DEV const uint16_t* rowc(int tok) const { return x + (int64_t)map[min(tok, rows - 1)] * ld; }
};

// Loads the A fragments of chunk c for tokens [tok0, tok0 + 16*XT).  Every
// lane issues its loads (clamped to a real token and block); mask_xfrags
// zeroes what lies past the tokens or k once the data is used, so neither the
// loads nor anything right after them waits on their data.
template <int FMT, int XT, class XS>
OCR_DEV void load_xfrags(const XS& xs, int tok0, int c, int nblk, int lane, half8v (&xa)[Geom<FMT>::SB][XT]) {
    constexpr int SB = Geom<FMT>::SB;
#pragma unroll
    for (int xt = 0; xt < XT; ++xt) {
        const uint16_t* p = xs.rowc(tok0 + 16 * xt + (lane & 15));
#pragma unroll
        for (int j = 0; j < SB; ++j)
            xa[j][xt] = bits_to_half8(*(const uint4*)(p + min(c * SB + j, nblk - 1) * 32 + 8 * (lane >> 4)));
    }
}

template <int FMT, int XT, class XS>
OCR_DEV void mask_xfrags(const XS& xs, int tok0, int c, int nblk, int lane, half8v (&xa)[Geom<FMT>::SB][XT]) {
    constexpr int SB = Geom<FMT>::SB;
    const half8v zero = {};
#pragma unroll
    for (int xt = 0; xt < XT; ++xt) {
        const bool tok_ok = tok0 + 16 * xt + (lane & 15) < xs.rows;
#pragma unroll
        for (int j = 0; j < SB; ++j)
            if (!(tok_ok && c * SB + j < nblk)) xa[j][xt] = zero;
    }
}

// Per-token sums of each block's activations (int8-asymmetric only): an MFMA
// against an all-ones B operand puts sum_k x[token][k] in every column.
template <int FMT, int XT>
OCR_DEV void xsums(const half8v (&xa)[Geom<FMT>::SB][XT], float4v (&xsum)[Geom<FMT>::SB][XT]) {
    if constexpr (FMT == OCRDEC_U8A_G32) {
        const half8v ones = {(f16_t)1, (f16_t)1, (f16_t)1, (f16_t)1, (f16_t)1, (f16_t)1, (f16_t)1, (f16_t)1};
        const float4v zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < Geom<FMT>::SB; ++j)
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) xsum[j][xt] = mfma16(xa[j][xt], ones, zero);
    }
}

// Prefetch depth that keeps the register ring near 96 VGPRs.
template <int FMT, int NT, int XT>
constexpr int kloop_depth() {
    constexpr int regs = NT * 6 + Geom<FMT>::SB * XT * 4;
    return regs * 4 <= 96 ? 4 : (regs * 3 <= 120 ? 3 : 2);
}

// The k-loop of one wavefront: NT tiles (tile[i] chunk pointers) over chunks
// [c0, c1), accumulating into acc[NT][XT].  A register ring keeps PF chunks
// in flight; each slot holds a chunk's weights AND its activation fragments,
// loaded together, so waiting for the oldest slot (vector loads complete in
// issue order) never waits for the younger prefetches.  The load of chunk
// c+PF is issued as soon as chunk c has been consumed.  The steady-state loop
// has no branches around its loads (the range is wavefront-uniform and the
// prologue reloads the last chunk when the range is shorter than the ring),
// so the compiler can wait for exactly the oldest slot instead of draining
// every load in flight.
template <int FMT, int NT, int XT, class XS, int PF = kloop_depth<FMT, NT, XT>()>
OCR_DEV void kloop(const uint8_t* const (&tile)[NT], int c0, int c1, const XS& xs, int tok0, int nblk, int lane,
                   float4v (&acc)[NT][XT]) {
    constexpr int CB = Geom<FMT>::CB;
    constexpr int SB = Geom<FMT>::SB;
    const int n = __builtin_amdgcn_readfirstlane(c1 - c0);
    const int cb = __builtin_amdgcn_readfirstlane(c0);
    if (n <= 0) return;
    q4_scale<FMT, NT, XT>(acc);
    WRegs wb[PF][NT];
    half8v xb[PF][SB][XT];
    auto fetch = [&](int u, int c) {
#pragma unroll
        for (int i = 0; i < NT; ++i) load_wchunk<FMT>(tile[i] + (int64_t)(cb + c) * CB, lane, wb[u][i]);
        load_xfrags<FMT, XT>(xs, tok0, cb + c, nblk, lane, xb[u]);
    };
    auto use = [&](int u, int c) {
        mask_xfrags<FMT, XT>(xs, tok0, cb + c, nblk, lane, xb[u]);
        float4v xsum[SB][XT];
        xsums<FMT, XT>(xb[u], xsum);
        chunk_mac_nt<FMT, NT, XT>(wb[u], xb[u], xsum, acc);
    };
#pragma unroll
    for (int u = 0; u < PF; ++u) fetch(u, min(u, n - 1));
    int it = 0;
    for (; it + 2 * PF <= n; it += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            use(u, it + u);
            fetch(u, it + u + PF);
            __builtin_amdgcn_sched_barrier(0);  // keep the slots in issue order
        }
    }
    // the last n - it chunks
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        if (it + u < n) {
            use(u, it + u);
            if (it + u + PF < n) fetch(u, it + u + PF);
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u)
        if (it + PF + u < n) use(u, it + PF + u);
    q4_unscale<FMT, NT, XT>(acc);
}

// ---------------------------------------------------------------------------
// LDS-staged activations
//
// The workgroup copies the activations of 16 or 32 tokens (zero rows past the
// token count) into LDS once per pass; every wavefront then reads its A
// fragments from LDS, so the k-loop streams only weights from memory.  Row
// stride ldl = k + 8 halves (16 bytes of padding shifts consecutive tokens by
// four banks).
// ---------------------------------------------------------------------------

OCR_DEV int xlds_stride(int k) { return k + 8; }

// Copies the activations of tokens tok0 .. tok0+ntok-1 (those that exist)
// into LDS.  The 16-byte pieces of all rows are spread over the workgroup's
// threads, and each thread issues up to B loads before it stores any: the
// copy takes one memory round trip per B pieces per thread instead of one
// per token row (for gathered rows, the row list is read first, in the same
// pass).  Fragments of the tokens not copied read as zero.
template <int B = 8, class XS>
OCR_DEV void stage_x(const XS& xs, int tok0, int ntok, int k, uint16_t* xl, int ldl) {
    const int nt = min(ntok, max(xs.rows - tok0, 0));
    const int n16 = k >> 3;  // 16-byte pieces per row
    const int total = nt * n16;
    const int nth = (int)blockDim.x, tid = (int)threadIdx.x;
    for (int b0 = 0; b0 < total; b0 += B * nth) {
        uint4 v[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int i = min(b0 + j * nth + tid, max(total - 1, 0));
            const int t = i / n16, c = i - t * n16;
            v[j] = total > 0 ? *(const uint4*)(xs.rowc(tok0 + t) + c * 8) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const int i = b0 + j * nth + tid;
            if (i < total) {
                const int t = i / n16, c = i - t * n16;
                *(uint4*)(xl + t * ldl + c * 8) = v[j];
            }
        }
    }
}

typedef __attribute__((address_space(3))) void lds_void_t;

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at their
// maxima, i.e. not waited for).
template <int N>
OCR_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Copies nt activation rows into LDS (row t at xl + t * ldl) with
// buffer loads that write LDS directly, no registers: wave w of the
// workgroup copies rows w, w + waves, ..., one instruction per 64 pieces of
// 16 bytes of a row.  row_of(t) gives row t's address (the same in every
// lane).  The caller waits for them (vmcnt) and then for the workgroup: issued
// ahead of the weights, they let the activations arrive first, as loads
// return in issue order.
template <class ROWF>
OCR_DEV void stage_rows_direct(ROWF row_of, int nt, int k, uint16_t* xl, int ldl) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int n16 = k >> 3;
    for (int t = wave; t < nt; t += nw) {
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc((void*)row_of(t), 0, 0x7fffffff, 0x00020000);
        for (int i = 0; 64 * i < n16; ++i)
            if (64 * i + lane < n16)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)(xl + t * ldl + 512 * i), 16, lane * 16,
                                                         1024 * i, 0, 0);
    }
}

// x = fp16(RMSNorm(h[r]) * gamma) for rows r0 .. r0+R-1 of the decode step's
// fixed-point residual (row stride H), formed by all waves of the workgroup
// into LDS (row r at xl + (r - r0) * ldl) and, if x_out is non-NULL, into
// x_out + r * ldx.  A wave holds at most MAXG four-value groups of a row per
// lane (8 * MAXG registers of raw residual), every load of them issued before
// the first use.  With few rows a row is cut into G slices, one per wave (up
// to four), whose partial sums of squares meet in LDS and are added in slice
// order (the result does not depend on timing); a wave with one slice keeps
// its values in registers, otherwise it reads its slices again (from cache)
// to scale them.  With G = 1 every wave normalises whole rows on its own.
// Every thread of the workgroup must call it (it may hold a barrier).
// Rows of fp16 embedding-table values, row r = table row tok[r] (clamped to
// [0, vocab)), read as the decode step's residual stores them: a non-finite
// value becomes 0 (the fixed-point residual holds every finite fp16 value
// exactly).  ETAB = nullptr: the rows are fixed-point residual rows.
struct EmbedRows {
    const uint16_t* table;
    const int32_t* tok;
    int vocab;
};
OCR_DEV int clamp_tok(int t, int vocab) { return t < 0 ? 0 : (t >= vocab ? vocab - 1 : t); }
OCR_DEV float embed_val(uint16_t b) {
    const float f = h2f(b);
    return fabsf(f) <= 65504.0f ? f : 0.0f;
}

template <int MAXG, bool EMB = false>
OCR_DEV void block_rmsnorm_fix(const fix_t* h, const uint16_t* gamma, int H, float eps, int r0, int R,
                               uint16_t* x_out, int64_t ldx, uint16_t* xl, int ldl, EmbedRows er = EmbedRows{}) {
    __shared__ float ss_lds[256];
    const int nw = (int)blockDim.x >> 6, wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
    const int n4 = H / 4;
    const int gmin = (n4 + 64 * MAXG - 1) / (64 * MAXG);
    const int G = max(gmin, min(4, nw / max(R, 1)));
    const int per = (n4 + G - 1) / G;
    const int np = R * G;
    const bool keep = np <= nw;
    float4 v[MAXG];
    uint2 g[MAXG];
    auto load = [&](int pr) {
        const int r = pr / G, s = pr % G;
        const int g0 = s * per, g1 = min(g0 + per, n4);
        if constexpr (EMB) {
            const int t = clamp_tok(er.tok[r0 + r], er.vocab);
            const uint2* er_row = (const uint2*)(er.table + (int64_t)t * H);
            uint2 e[MAXG];
#pragma unroll
            for (int i = 0; i < MAXG; ++i) {
                const int c = min(g0 + lane + 64 * i, g1 - 1);
                e[i] = er_row[c];
                g[i] = ((const uint2*)gamma)[c];
            }
#pragma unroll
            for (int i = 0; i < MAXG; ++i)
                v[i] = g0 + lane + 64 * i < g1
                           ? make_float4(embed_val((uint16_t)(e[i].x & 0xFFFF)), embed_val((uint16_t)(e[i].x >> 16)),
                                         embed_val((uint16_t)(e[i].y & 0xFFFF)), embed_val((uint16_t)(e[i].y >> 16)))
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
            const fix_t* hr = h + (int64_t)(r0 + r) * H;
            longlong2 a[MAXG], b[MAXG];
#pragma unroll
            for (int i = 0; i < MAXG; ++i) {
                const int c = min(g0 + lane + 64 * i, g1 - 1);
                a[i] = ((const longlong2*)hr)[2 * c];
                b[i] = ((const longlong2*)hr)[2 * c + 1];
                g[i] = ((const uint2*)gamma)[c];
            }
#pragma unroll
            for (int i = 0; i < MAXG; ++i)
                v[i] = g0 + lane + 64 * i < g1
                           ? make_float4(fix_to(a[i].x), fix_to(a[i].y), fix_to(b[i].x), fix_to(b[i].y))
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    auto sumsq = [&]() {
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < MAXG; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
        return wave_sum(ss);
    };
    auto scale = [&](int pr, float tot) {
        const int r = pr / G, s = pr % G;
        const float inv = 1.0f / sqrtf(tot / (float)H + eps);
        const int g0 = s * per, g1 = min(g0 + per, n4);
#pragma unroll
        for (int i = 0; i < MAXG; ++i) {
            const int c4 = g0 + lane + 64 * i;
            if (c4 < g1) {
                const uint32_t lo = (uint32_t)f2h(v[i].x * inv * h2f((uint16_t)(g[i].x & 0xFFFF))) |
                                    ((uint32_t)f2h(v[i].y * inv * h2f((uint16_t)(g[i].x >> 16))) << 16);
                const uint32_t hi = (uint32_t)f2h(v[i].z * inv * h2f((uint16_t)(g[i].y & 0xFFFF))) |
                                    ((uint32_t)f2h(v[i].w * inv * h2f((uint16_t)(g[i].y >> 16))) << 16);
                ((uint2*)(xl + r * ldl))[c4] = make_uint2(lo, hi);
                if (x_out) ((uint2*)(x_out + (int64_t)(r0 + r) * ldx))[c4] = make_uint2(lo, hi);
            }
        }
    };
    if (G == 1) {  // whole rows per wave: no exchange
        for (int pr = wave; pr < np; pr += nw) {
            load(pr);
            scale(pr, sumsq());
        }
        return;
    }
    for (int pr = wave; pr < np; pr += nw) {
        load(pr);
        const float ss = sumsq();
        if (lane == 0) ss_lds[pr] = ss;
    }
    __syncthreads();
    for (int pr = wave; pr < np; pr += nw) {
        if (!keep) load(pr);
        const int r = pr / G;
        float tot = 0.f;
        for (int j = 0; j < G; ++j) tot += ss_lds[r * G + j];
        scale(pr, tot);
    }
}

// block_rmsnorm_fix for one row, in two phases for a kernel that also
// requests weights: issue() requests row r0's slices (wave w < G takes slice
// w of G) as raw fixed-point values and gains in registers, finish() forms
// the norm (partial sums of squares added in slice order in LDS, as
// block_rmsnorm_fix does) into LDS row 0 and x_out row r0.  The workgroup
// must have at least G wavefronts; every thread calls both.
template <int MAXG>
struct RowNormFix {
    longlong2 a[MAXG], b[MAXG];
    uint2 g[MAXG];
    int G, per, n4, g0, g1;
    OCR_DEV void issue(const fix_t* h, const uint16_t* gamma, int H, int r0) {
        const int nw = (int)blockDim.x >> 6, wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
        n4 = H / 4;
        const int gmin = (n4 + 64 * MAXG - 1) / (64 * MAXG);
        G = max(gmin, min(4, nw));
        per = (n4 + G - 1) / G;
        const int sl = min(wave, G - 1);
        g0 = sl * per;
        g1 = min(g0 + per, n4);
        const fix_t* hr = h + (int64_t)r0 * H;
        if (wave < G) {
#pragma unroll
            for (int i = 0; i < MAXG; ++i) {
                const int c = min(g0 + lane + 64 * i, g1 - 1);
                a[i] = ((const longlong2*)hr)[2 * c];
                b[i] = ((const longlong2*)hr)[2 * c + 1];
                g[i] = ((const uint2*)gamma)[c];
            }
        }
    }
    OCR_DEV void finish(int H, float eps, int r0, uint16_t* x_out, int64_t ldx, uint16_t* xl) {
        __shared__ float ss_lds[16];
        const int wave = (int)threadIdx.x >> 6, lane = (int)threadIdx.x & 63;
        float4 v[MAXG];
#pragma unroll
        for (int i = 0; i < MAXG; ++i)
            v[i] = wave < G && g0 + lane + 64 * i < g1
                       ? make_float4(fix_to(a[i].x), fix_to(a[i].y), fix_to(b[i].x), fix_to(b[i].y))
                       : make_float4(0.f, 0.f, 0.f, 0.f);
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < MAXG; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
        ss = wave_sum(ss);
        if (lane == 0 && wave < G) ss_lds[wave] = ss;
        __syncthreads();
        if (wave < G) {
            float tot = 0.f;
            for (int j = 0; j < G; ++j) tot += ss_lds[j];
            const float inv = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
            for (int i = 0; i < MAXG; ++i) {
                const int c4 = g0 + lane + 64 * i;
                if (c4 < g1) {
                    const uint32_t lo = (uint32_t)f2h(v[i].x * inv * h2f((uint16_t)(g[i].x & 0xFFFF))) |
                                        ((uint32_t)f2h(v[i].y * inv * h2f((uint16_t)(g[i].x >> 16))) << 16);
                    const uint32_t hi = (uint32_t)f2h(v[i].z * inv * h2f((uint16_t)(g[i].y & 0xFFFF))) |
                                        ((uint32_t)f2h(v[i].w * inv * h2f((uint16_t)(g[i].y >> 16))) << 16);
                    ((uint2*)xl)[c4] = make_uint2(lo, hi);
                    if (x_out) ((uint2*)(x_out + (int64_t)r0 * ldx))[c4] = make_uint2(lo, hi);
                }
            }
        }
    }
};

// x = fp16(RMSNorm(h[tok]) * gamma) for tokens tok0 .. tok0+15 of rows into
// LDS (row stride ldl); tokens past the row count are not written (their
// fragments read as zero).  All threads of the workgroup call it.
OCR_DEV void stage_norm(const fix_t* h, const uint16_t* gamma, float eps, int rows, int tok0, int H, uint16_t* xl,
                        int ldl) {
    block_rmsnorm_fix<5>(h, gamma, H, eps, tok0, min(16, rows - tok0), nullptr, 0, xl, ldl);
}
// The same from embedding rows (first layer of the decode step).
OCR_DEV void stage_embed_norm(EmbedRows er, const uint16_t* gamma, float eps, int rows, int tok0, int H,
                              uint16_t* xl, int ldl) {
    block_rmsnorm_fix<5, true>(nullptr, gamma, H, eps, tok0, min(16, rows - tok0), nullptr, 0, xl, ldl, er);
}

template <int FMT, int XT>
OCR_DEV void lds_xfrags(const uint16_t* xl, int ldl, int ntok, int c, int nblk, int lane,
                        half8v (&xa)[Geom<FMT>::SB][XT]) {
#pragma unroll
    for (int xt = 0; xt < XT; ++xt)
#pragma unroll
        for (int j = 0; j < Geom<FMT>::SB; ++j) {
            const int blk = c * Geom<FMT>::SB + j;
            const int tok = 16 * xt + (lane & 15);
            uint4 v = make_uint4(0, 0, 0, 0);
            if (blk < nblk && tok < ntok) v = *(const uint4*)(xl + tok * ldl + blk * 32 + 8 * (lane >> 4));
            xa[j][xt] = bits_to_half8(v);
        }
}

// lds_xfrags without range checks, for a k of whole chunks: the LDS rows past
// the token count hold stale values, which reach only those tokens' outputs
// (an MFMA output row depends on its own A row alone), and those are never
// stored.
template <int FMT>
OCR_DEV void lds_xfrags_all(const uint16_t* xl, int ldl, int c, int lane, half8v (&xa)[Geom<FMT>::SB][1]) {
#pragma unroll
    for (int j = 0; j < Geom<FMT>::SB; ++j)
        xa[j][0] = bits_to_half8(
            *(const uint4*)(xl + (lane & 15) * ldl + (c * Geom<FMT>::SB + j) * 32 + 8 * (lane >> 4)));
}

template <int FMT, int NT>
constexpr int kloop_lds_depth() {
    return NT * 6 * 6 <= 72 ? 6 : (NT * 6 * 4 <= 96 ? 4 : 3);
}

// k-loop over LDS-staged activations (16*XT tokens).  The weight ring's first
// PF chunks are requested before the activations are staged (stage() copies
// them into LDS; the barrier follows), so both travel in the same round trip;
// afterwards the A fragments come from LDS and only weights stream from
// memory.
struct NoIssue {
    OCR_DEV void operator()() const {}
};

// Weight load instructions of a kloop_lds prologue (its PF chunks of NT tiles).
template <int FMT, int NT, int PF>
constexpr int kloop_prologue_loads() { return PF * NT * (FMT == OCRDEC_F16 ? 1 : 2); }

// pre(), if given: runs before the first weight chunks are requested
// (activation loads issued there travel ahead of the weights); stage() after
// them.  With pre() the first PF chunks are requested unconditionally (a
// short range repeats its last chunk; an empty one reads a chunk of the tile
// in range: c0 <= nchunks and c1 <= nchunks), so that exactly
// kloop_prologue_loads() loads follow pre().
template <int FMT, int NT, int XT, class STAGE, int PF = kloop_lds_depth<FMT, NT>(), class PRE = NoIssue>
OCR_DEV void kloop_lds(const uint8_t* const (&tile)[NT], int c0, int c1, STAGE stage, const uint16_t* xl, int ldl,
                       int ntok, int nblk, int lane, float4v (&acc)[NT][XT], PRE pre = PRE{}) {
    constexpr int CB = Geom<FMT>::CB;
    constexpr int SB = Geom<FMT>::SB;
    constexpr bool PRE_ISSUES = !std::is_same<PRE, NoIssue>::value;
    pre();
    if constexpr (PRE_ISSUES) __builtin_amdgcn_sched_barrier(0);
    WRegs wb[PF][NT];
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        if constexpr (PRE_ISSUES) {
            const int cu = max(min(c0 + u, c1 - 1), 0);
#pragma unroll
            for (int i = 0; i < NT; ++i) load_wchunk<FMT>(tile[i] + (int64_t)cu * CB, lane, wb[u][i]);
        } else if (c0 + u < c1) {
#pragma unroll
            for (int i = 0; i < NT; ++i) load_wchunk<FMT>(tile[i] + (int64_t)(c0 + u) * CB, lane, wb[u][i]);
        }
    }
    if constexpr (PRE_ISSUES) __builtin_amdgcn_sched_barrier(0);
    stage();
    __syncthreads();
    q4_scale<FMT, NT, XT>(acc);
    for (int c = c0; c < c1; c += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int cc = c + u;
            if (cc < c1) {
                half8v xa[SB][XT];
                float4v xsum[SB][XT];
                lds_xfrags<FMT, XT>(xl, ldl, ntok, cc, nblk, lane, xa);
                xsums<FMT, XT>(xa, xsum);
                chunk_mac_nt<FMT, NT, XT>(wb[u], xa, xsum, acc);
                if (cc + PF < c1) {
#pragma unroll
                    for (int i = 0; i < NT; ++i)
                        load_wchunk<FMT>(tile[i] + (int64_t)(cc + PF) * CB, lane, wb[u][i]);
                }
            }
        }
    }
    q4_unscale<FMT, NT, XT>(acc);
}

// LDS bytes for 16*xt tokens of k activations.  The LDS path is used when it
// fits in 64 KiB and there are enough tokens to pay for the staging (with 1-3
// tokens the fragments are cheaper to load alongside the weights).
inline size_t lds_x_bytes(int k, int xt) { return (size_t)16 * xt * (k + 8) * 2; }
inline bool use_lds_x(int k, int xt, int rows) { return rows >= 4 && lds_x_bytes(k, xt) <= 65536; }

// Sums the accumulators of the KS waves that share a tile group (waves
// g*KS .. g*KS+KS-1 of the workgroup) in a fixed order; the result is valid in
// the first of them.  red: LDS scratch of 4 * NT * XT * 64 float4v.
template <int NT, int XT, int KS>
OCR_DEV void ksplit_reduce(float4v (&acc)[NT][XT], float4v* red, int wave, int lane) {
    if constexpr (KS == 1) return;
    const int ks = wave % KS;
    if (ks != 0) {
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) red[((wave * NT + i) * XT + xt) * 64 + lane] = acc[i][xt];
    }
    __syncthreads();
    if (ks == 0) {
        for (int o = 1; o < KS; ++o) {
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int xt = 0; xt < XT; ++xt) acc[i][xt] += red[(((wave + o) * NT + i) * XT + xt) * 64 + lane];
        }
    }
}

}  // namespace ocrdec

// Dense GEMV / skinny-GEMM kernels over packed weights, with the epilogues the
// decode step needs: fp32 or fp16 store, residual add, SwiGLU pairing, and a
// fused argmax over the output rows (language head).
#include "gemv.hpp"

namespace ocrdec {

// XT = 1, 2: 16 or 32 tokens per pass.  XSRC: where the activations come
// from: X_GLOBAL, their fragments are loaded from global memory alongside the
// weights (for k too large to stage); X_LDS, they are staged in LDS;
// X_NORM (XT = 1), formed in LDS as RMSNorm(hn) * gamma; X_EMBED (XT = 1,
// one pass), the same from embedding rows (GemvParams::er).
constexpr int X_GLOBAL = 0, X_LDS = 1, X_NORM = 2, X_EMBED = 3;
template <int FMT, int NT, int XT, int KS, int EPI, int XSRC>
__global__ __launch_bounds__(256) void gemv_kernel(GemvParams p) {
    constexpr int CB = Geom<FMT>::CB;
    extern __shared__ __align__(16) uint16_t xl_dyn[];
    __shared__ float4v red[(KS > 1) ? 4 * NT * XT * 64 : 1];
    __shared__ float amx[(EPI == EPI_ARGMAX) ? 4 * 32 * 3 : 1];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = blockIdx.x * (4 / KS) + wave / KS;
    const int ks = wave % KS;
    const bool valid = g < p.n_groups;
    const int ntiles = (p.n + 15) / 16;

    int tidx[NT];
    const uint8_t* tile[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        int t = (EPI == EPI_GLU) ? (i == 0 ? g : g + p.half_tiles) : g * NT + i;
        tidx[i] = t;
        if (!valid || t >= ntiles) t = 0;
        tile[i] = p.w + (int64_t)t * p.nchunks * CB;
    }
    const int cper = (int)((p.nchunks + KS - 1) / KS);
    const int c0 = ks * cper;
    const int c1 = valid ? (int)min((int64_t)(c0 + cper), p.nchunks) : c0;
    const int nblk = p.k / 32;

    const int ldl = xlds_stride(p.k);
    for (int tok0 = 0; tok0 < p.xs.rows; tok0 += 16 * XT) {
        float4v acc[NT][XT];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) acc[i][xt] = float4v{0.f, 0.f, 0.f, 0.f};
        // residual epilogue: the residual values are requested now, so that
        // the add does not wait a memory round trip after the k-loop (every
        // output element belongs to one workgroup: nobody else writes it)
        fix_t hpre[(EPI == EPI_RESID) ? NT : 1][(EPI == EPI_RESID) ? XT : 1][4];
        if constexpr (EPI == EPI_RESID) {
            const fix_t* h = (const fix_t*)p.y;
#pragma unroll
            for (int i = 0; i < NT; ++i)
#pragma unroll
                for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int tok = tok0 + 16 * xt + 4 * (lane >> 4) + v;
                        const int row = tidx[i] * 16 + (lane & 15);
                        const bool in = ks == 0 && valid && tok < p.xs.rows && row < p.n;
                        hpre[i][xt][v] = in ? h[(int64_t)tok * p.ldy + row] : 0;
                    }
        }
        if constexpr (XSRC != X_GLOBAL) {
            auto stage = [&]() {
                if constexpr (XSRC == X_NORM) stage_norm(p.hn, p.gamma, p.eps, p.xs.rows, tok0, p.k, xl_dyn, ldl);
                else if constexpr (XSRC == X_EMBED)
                    stage_embed_norm(p.er, p.gamma, p.eps, p.xs.rows, tok0, p.k, xl_dyn, ldl);
                else stage_x(p.xs, tok0, 16 * XT, p.k, xl_dyn, ldl);
            };
            kloop_lds<FMT, NT, XT>(tile, c0, c1, stage, xl_dyn, ldl, p.xs.rows - tok0, nblk, lane, acc);
        } else {
            kloop<FMT, NT, XT>(tile, c0, c1, p.xs, tok0, nblk, lane, acc);
        }
        ksplit_reduce<NT, XT, KS>(acc, red, wave, lane);

        const bool owner = (ks == 0) && valid;
        if constexpr (EPI == EPI_ARGMAX) {
            // per token: best value, its row (lowest on ties), second-best value
            float best[XT][4], second[XT][4];
            int bidx[XT][4];
            bool nonfin = false;
#pragma unroll
            for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    best[xt][v] = -INFINITY;
                    second[xt][v] = -INFINITY;
                    bidx[xt][v] = 0x7fffffff;
                }
            if (owner) {
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    const int row = tidx[i] * 16 + (lane & 15);
                    if (row < p.n) {
#pragma unroll
                        for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                float val = acc[i][xt][v];
                                nonfin |= !(fabsf(val) < INFINITY);
                                if (val > best[xt][v]) {
                                    second[xt][v] = best[xt][v];
                                    best[xt][v] = val;
                                    bidx[xt][v] = row;
                                } else if (val > second[xt][v]) {
                                    second[xt][v] = val;
                                }
                            }
                    }
                }
            }
            // merge across the 16 lanes that share a token
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) {
#pragma unroll
                for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        float ob = __shfl_xor(best[xt][v], o, 64);
                        float os = __shfl_xor(second[xt][v], o, 64);
                        int oi = __shfl_xor(bidx[xt][v], o, 64);
                        argmax_merge(best[xt][v], bidx[xt][v], second[xt][v], ob, oi, os);
                    }
            }
            if ((lane & 15) == 0) {
#pragma unroll
                for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int tok = 16 * xt + 4 * (lane >> 4) + v;
                        float* e = amx + (wave * 32 + tok) * 3;
                        e[0] = best[xt][v];
                        e[1] = __int_as_float(bidx[xt][v]);
                        e[2] = second[xt][v];
                    }
            }
            // a non-finite logit anywhere in the workgroup is recorded with
            // every token's partial (the final merge ORs the flags)
            const int wg_nonfin = __syncthreads_or(nonfin ? 1 : 0);
            if (threadIdx.x < 16 * XT) {
                const int tok = threadIdx.x;
                float b = -INFINITY, s = -INFINITY;
                int bi = 0x7fffffff;
                for (int w = 0; w < 4; ++w) {
                    const float* e = amx + (w * 32 + tok) * 3;
                    argmax_merge(b, bi, s, e[0], __float_as_int(e[1]), e[2]);
                }
                if (tok0 + tok < p.xs.rows) {
                    float* out = p.part + ((int64_t)blockIdx.x * p.xs.rows + tok0 + tok) * 4;
                    out[0] = b;
                    out[1] = __int_as_float(bi);
                    out[2] = s;
                    out[3] = __int_as_float(wg_nonfin ? (int)kStatLogit : 0);
                }
            }
        } else {
            bool bad = false;
            if (owner) {
#pragma unroll
            for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int tok = tok0 + 16 * xt + 4 * (lane >> 4) + v;
                    if (tok >= p.xs.rows) continue;
                    if constexpr (EPI == EPI_GLU) {
                        const int col = tidx[0] * 16 + (lane & 15);
                        if (col < p.half_tiles * 16) {
                            const float gv = acc[0][xt][v], uv = acc[1][xt][v];
                            ((uint16_t*)p.y)[(int64_t)tok * p.ldy + col] = f2h(silu(gv) * uv);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < NT; ++i) {
                            const int row = tidx[i] * 16 + (lane & 15);
                            if (row >= p.n) continue;
                            const int64_t o = (int64_t)tok * p.ldy + row;
                            if constexpr (EPI == EPI_F32) {
                                ((float*)p.y)[o] = acc[i][xt][v];
                            } else if constexpr (EPI == EPI_F16) {
                                ((uint16_t*)p.y)[o] = f2h(acc[i][xt][v]);
                            } else if constexpr (EPI == EPI_RESID) {
                                ((fix_t*)p.y)[o] = hpre[i][xt][v] + fix_from(acc[i][xt][v], bad);
                            }
                        }
                    }
                }
            }
            if constexpr (EPI == EPI_RESID) report_status(p.status, bad, kStatResidual);
        }
        __syncthreads();
    }
    if constexpr (XSRC == X_EMBED) {
        // workgroup b stores embedding rows b, b + grid, ... into the
        // residual (a non-finite value is stored as 0 and flagged) and opens
        // their status words
        __shared__ int bad_s;
        for (int r = blockIdx.x; r < p.xs.rows; r += gridDim.x) {
            if (threadIdx.x == 0) bad_s = 0;
            __syncthreads();
            const int t0 = p.er.tok[r];
            const bool tok_bad = t0 < 0 || t0 >= p.er.vocab;
            const uint2* er_row = (const uint2*)(p.er.table + (int64_t)clamp_tok(t0, p.er.vocab) * p.k);
            fix_t* hr = p.eh + (int64_t)r * p.k;
            bool bad = false;
            for (int c4 = threadIdx.x; c4 < p.k / 4; c4 += blockDim.x) {
                const uint2 e = er_row[c4];
                st_resid4(hr, c4,
                          make_float4(h2f((uint16_t)(e.x & 0xFFFF)), h2f((uint16_t)(e.x >> 16)),
                                      h2f((uint16_t)(e.y & 0xFFFF)), h2f((uint16_t)(e.y >> 16))),
                          bad);
            }
            if (__ballot(bad) != 0 && lane == 0) atomicOr(&bad_s, 1);
            __syncthreads();
            if (wave == 0) status_begin(p.status, r, p.xs.rows, tok_bad, bad_s != 0);
        }
    }
}

namespace {

template <int FMT, int NT, int XT, int KS, int EPI, int XSRC>
void launch_t(const GemvParams& p, hipStream_t s) {
    const int groups_per_wg = 4 / KS;
    const int grid = (p.n_groups + groups_per_wg - 1) / groups_per_wg;
    const size_t lds = XSRC != X_GLOBAL ? lds_x_bytes(p.k, XT) : 0;
    hipLaunchKernelGGL((gemv_kernel<FMT, NT, XT, KS, EPI, XSRC>), dim3(grid), dim3(256), lds, s, p);
}

template <int FMT, int EPI>
void launch_fmt(const GemvParams& p, int nt, int ks, int xt, int xsrc, hipStream_t s) {
#define OCR_L(NT_, KS_, XT_)                                                                 \
    if (nt == NT_ && ks == KS_ && xt == XT_) {                                               \
        if constexpr (XT_ == 1)                                                              \
            if (xsrc == X_NORM) return launch_t<FMT, NT_, XT_, KS_, EPI, X_NORM>(p, s);       \
        if constexpr (XT_ == 1 && EPI == EPI_F32)                                            \
            if (xsrc == X_EMBED) return launch_t<FMT, NT_, XT_, KS_, EPI, X_EMBED>(p, s);     \
        if (xsrc == X_LDS) launch_t<FMT, NT_, XT_, KS_, EPI, X_LDS>(p, s);                   \
        else launch_t<FMT, NT_, XT_, KS_, EPI, X_GLOBAL>(p, s);                              \
        return;                                                                              \
    }
    if constexpr (EPI == EPI_GLU) {
        OCR_L(2, 1, 1) OCR_L(2, 1, 2) OCR_L(2, 4, 1) OCR_L(2, 4, 2)
    } else {
        OCR_L(1, 4, 1) OCR_L(1, 4, 2) OCR_L(4, 1, 1) OCR_L(4, 1, 2)
    }
#undef OCR_L
}

}  // namespace

GemvPlan plan_gemv(int fmt, int n, int k, int rows, int epi) {
    GemvPlan pl;
    const int64_t tiles = (n + 15) / 16;
    pl.xt = rows <= 16 ? 1 : 2;
    pl.lds = use_lds_x(k, pl.xt, rows);
    if (epi == EPI_GLU) {
        pl.nt = 2;
        pl.groups = (int)(tiles / 2);
        pl.ks = pl.groups >= 512 ? 1 : 4;
    } else if (tiles >= 1024) {
        pl.nt = 4;
        pl.ks = 1;
        pl.groups = (int)((tiles + 3) / 4);
    } else {
        pl.nt = 1;
        pl.ks = 4;
        pl.groups = (int)tiles;
    }
    pl.grid = (pl.groups + (4 / pl.ks) - 1) / (4 / pl.ks);
    (void)fmt;
    (void)k;
    return pl;
}

void launch_gemv(int fmt, int epi, const GemvPlan& plan, GemvParams p, hipStream_t s) {
    // forming the activations from the residual needs the LDS staging and
    // 16-token passes
    GemvPlan pl = plan;
    if (p.hn) pl.xt = 1;
    const int xsrc = p.hn ? (p.er.table ? X_EMBED : X_NORM) : (pl.lds ? X_LDS : X_GLOBAL);
    p.n_groups = pl.groups;
#define OCR_E(E_)                                                                          \
    case E_:                                                                               \
        switch (fmt) {                                                                     \
        case OCRDEC_F16: launch_fmt<OCRDEC_F16, E_>(p, pl.nt, pl.ks, pl.xt, xsrc, s); break;     \
        case OCRDEC_Q8_0: launch_fmt<OCRDEC_Q8_0, E_>(p, pl.nt, pl.ks, pl.xt, xsrc, s); break;   \
        case OCRDEC_Q4_0: launch_fmt<OCRDEC_Q4_0, E_>(p, pl.nt, pl.ks, pl.xt, xsrc, s); break;   \
        case OCRDEC_U8A_G32: launch_fmt<OCRDEC_U8A_G32, E_>(p, pl.nt, pl.ks, pl.xt, xsrc, s); break; \
        }                                                                                  \
        break;
    switch (epi) {
        OCR_E(EPI_F32)
        OCR_E(EPI_F16)
        OCR_E(EPI_RESID)
        OCR_E(EPI_GLU)
        OCR_E(EPI_ARGMAX)
    }
#undef OCR_E
}

size_t argmax_ws_bytes(int grid, int rows) { return align256((size_t)grid * rows * 4 * sizeof(float)); }

// ---------------------------------------------------------------------------
// LM head with fused argmax for up to 16 rows, balanced within each CU
//
// One workgroup of eight wavefronts (twelve for Q4_0, U8A) per CU (its LDS
// request leaves room for no second one) owns an equal slice of the 16-row
// tiles.  Its wavefronts
// take tiles one at a time from an LDS counter, so a wavefront the CU favours
// (the issue arbiter prefers older waves) simply takes more tiles, and all of
// a CU's wavefronts finish within about one tile of each other.  Each
// wavefront streams its tiles as one chunk sequence through a ring of PF
// chunks: the ring runs on into the next tile's first chunks while the
// current tile finishes.  The activations (<= 16 rows) are staged in LDS
// once.  Per tile the 16 dot products of every row update a running (best,
// index, second) per lane; the workgroup's partial goes to part[blockIdx.x].
// ---------------------------------------------------------------------------

constexpr int LM_WAVES = 8;
constexpr size_t LM_LDS = 96 * 1024;  // > half the CU's LDS: one workgroup per CU

// Wavefronts per workgroup: eight, twelve for Q4_0 and U8A (their rings of
// five chunks hold a sixth of an fp16 ring's bytes, and three waves per SIMD
// fit their registers; sixteen Q8_0 wavefronts measured no faster than eight)
template <int FMT>
constexpr int lm_waves() { return FMT == OCRDEC_Q4_0 || FMT == OCRDEC_U8A_G32 ? 12 : LM_WAVES; }

template <int FMT, int PF>
__global__ __launch_bounds__(64 * lm_waves<FMT>(), 1) void lm_argmax_kernel(GemvParams p) {
    constexpr int SB = Geom<FMT>::SB, CB = Geom<FMT>::CB;
    constexpr int NWV = lm_waves<FMT>();
    extern __shared__ __align__(16) uint16_t xl_dyn[];
    __shared__ float amx[NWV * 16 * 3];
    __shared__ int next_s;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ntiles = (p.n + 15) / 16;
    const int t0 = (int)((int64_t)ntiles * blockIdx.x / gridDim.x);
    const int nt = (int)((int64_t)ntiles * (blockIdx.x + 1) / gridDim.x) - t0;
    const int nc = (int)p.nchunks, nblk = p.k / 32, ldl = xlds_stride(p.k), R = p.xs.rows;
    // tiles of the slice: wave w starts with tile w, then asks the counter
    if (threadIdx.x == 0) next_s = NWV;
    auto tptr = [&](int u) { return p.w + (int64_t)(t0 + min(u, max(nt - 1, 0))) * nc * CB; };
    WRegs ring[PF];
    int ucur = wave;
#pragma unroll
    for (int s = 0; s < PF; ++s) load_wchunk<FMT>(tptr(ucur) + (int64_t)s * CB, lane, ring[s]);
    if (p.hn) stage_norm(p.hn, p.gamma, p.eps, R, 0, p.k, xl_dyn, ldl);
    else stage_x(p.xs, 0, 16, p.k, xl_dyn, ldl);
    __syncthreads();
    float* btab = (float*)(xl_dyn + 16 * ldl);  // Q4_0: the blocks' accumulator inputs, after the rows
    if constexpr (FMT == OCRDEC_Q4_0) {
        q4_split_prepare(xl_dyn, ldl, R, nblk, nc * 4, btab);
        __syncthreads();
    }
    auto grab = [&]() {
        int u = 0;
        if (lane == 0) u = atomicAdd(&next_s, 1);
        return __builtin_amdgcn_readfirstlane(u);
    };
    int unxt = grab();
    float best[4], second[4];
    int bidx[4];
    bool nonfin = false;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        best[v] = -INFINITY;
        second[v] = -INFINITY;
        bidx[v] = 0x7fffffff;
    }
    while (ucur < nt) {  // uniform per wavefront
        const int unn = unxt < nt ? grab() : unxt;  // the tile after the next, asked for early
        const uint8_t* tc = tptr(ucur);
        const uint8_t* tn = tptr(unxt);
        float4v acc[1][1] = {{float4v{0.f, 0.f, 0.f, 0.f}}};
        for (int c0 = 0; c0 < nc; c0 += PF) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                const int c = c0 + s;
                half8v xa[SB][1];
                float4v xs[SB][1];
                // Q4_0 (whole chunks only): unchecked reads; the LDS rows past
                // the token count hold stale values that reach only those
                // tokens' outputs, which are never reported
                if constexpr (FMT == OCRDEC_Q4_0) lds_xfrags_all<FMT>(xl_dyn, ldl, c, lane, xa);
                else lds_xfrags<FMT, 1>(xl_dyn, ldl, R, c, nblk, lane, xa);
                if constexpr (FMT == OCRDEC_Q4_0) {
                    float4v nb[4][1];
#pragma unroll
                    for (int j = 0; j < 4; ++j) nb[j][0] = *(const float4v*)(btab + 16 * (4 * c + j) + 4 * (lane >> 4));
                    chunk_mac_q4b<1, 1, true>(&ring[s], xa, nb, acc);
                } else {
                    xsums<FMT, 1>(xa, xs);
                    chunk_mac<FMT, 1>(ring[s], xa, xs, acc[0]);
                }
                // refill the slot with the chunk PF further on in the stream
                // (the next tile's, past this one's end; nc % PF == 0)
                const int cf = c + PF;
                load_wchunk<FMT>(cf < nc ? tc + (int64_t)cf * CB : tn + (int64_t)(cf - nc) * CB, lane, ring[s]);
            }
        }
        if constexpr (FMT == OCRDEC_Q4_0) scale_acc<1, 1>(acc, Q4_RAW_SCALE);  // (raw codes)
        const int row = (t0 + ucur) * 16 + (lane & 15);
        if (row < p.n) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float val = acc[0][0][v];
                nonfin |= 4 * (lane >> 4) + v < R && !(fabsf(val) < INFINITY);
                if (val > best[v]) {
                    second[v] = best[v];
                    best[v] = val;
                    bidx[v] = row;
                } else if (val > second[v]) {
                    second[v] = val;
                }
            }
        }
        ucur = unxt;
        unxt = unn;
    }
    // merge across the 16 lanes that share a token, then across the wavefronts
#pragma unroll
    for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float ob = __shfl_xor(best[v], o, 64), os = __shfl_xor(second[v], o, 64);
            const int oi = __shfl_xor(bidx[v], o, 64);
            argmax_merge(best[v], bidx[v], second[v], ob, oi, os);
        }
    if ((lane & 15) == 0) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float* e = amx + (wave * 16 + 4 * (lane >> 4) + v) * 3;
            e[0] = best[v];
            e[1] = __int_as_float(bidx[v]);
            e[2] = second[v];
        }
    }
    const int wg_nonfin = __syncthreads_or(nonfin ? 1 : 0);
    if ((int)threadIdx.x < R) {
        const int tok = threadIdx.x;
        float b = -INFINITY, s2 = -INFINITY;
        int bi = 0x7fffffff;
        for (int w = 0; w < NWV; ++w) {
            const float* e = amx + (w * 16 + tok) * 3;
            argmax_merge(b, bi, s2, e[0], __float_as_int(e[1]), e[2]);
        }
        float* out = p.part + ((int64_t)blockIdx.x * R + tok) * 4;
        out[0] = b;
        out[1] = __int_as_float(bi);
        out[2] = s2;
        out[3] = __int_as_float(wg_nonfin ? (int)kStatLogit : 0);
    }
}

namespace {
int device_cus() {
    static int cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (!cus[dev]) {
        int c = 0;
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
        cus[dev] = c;
    }
    return cus[dev];
}
// ring depth in chunks: ~10 KiB per wavefront in flight; the chunk count of
// a row must be a multiple of it (0: not supported, the general GEMV runs)
int lm_pf(int fmt, int k) {
    const int64_t nc = n_chunks(fmt, k);
    if (fmt == OCRDEC_F16) return nc % 10 == 0 ? 10 : nc % 8 == 0 ? 8 : 0;
    if (fmt == OCRDEC_Q4_0 && k % 128 != 0) return 0;  // its unchecked operand reads need whole chunks
    return nc % 5 == 0 ? 5 : nc % 4 == 0 ? 4 : 0;
}
}  // namespace

LmPlan plan_lm(int fmt, int n, int k, int rows) {
    LmPlan lp;
    const int pf = lm_pf(fmt, k);
    const int ntiles = (n + 15) / 16;
    // the staged activations (row stride k + 8), then for Q4_0 16 floats per
    // 32-column block of the padded k range
    const size_t xb = (size_t)16 * (k + 8) * 2 + (fmt == OCRDEC_Q4_0 ? (size_t)n_chunks(fmt, k) * 4 * 64 : 0);
    lp.dyn = rows <= 16 && pf > 0 && xb <= LM_LDS && ntiles >= 8 * device_cus();
    lp.grid = lp.dyn ? device_cus() : plan_gemv(fmt, n, k, rows, EPI_ARGMAX).grid;
    return lp;
}

void launch_lm_argmax(int fmt, const LmPlan& lp, GemvParams p, hipStream_t s) {
    if (!lp.dyn) {
        const GemvPlan pl = plan_gemv(fmt, p.n, p.k, p.xs.rows, EPI_ARGMAX);
        launch_gemv(fmt, EPI_ARGMAX, pl, p, s);
        return;
    }
    const int pf = lm_pf(fmt, p.k);
#define OCR_LM(F_, A_, B_)                                                                                      \
    case F_:                                                                                                    \
        if (pf == A_)                                                                                           \
            hipLaunchKernelGGL((lm_argmax_kernel<F_, A_>), dim3(lp.grid), dim3(64 * lm_waves<F_>()), LM_LDS, s, p);    \
        else                                                                                                    \
            hipLaunchKernelGGL((lm_argmax_kernel<F_, B_>), dim3(lp.grid), dim3(64 * lm_waves<F_>()), LM_LDS, s, p);    \
        break;
    switch (fmt) {
        OCR_LM(OCRDEC_F16, 10, 8)
        OCR_LM(OCRDEC_Q8_0, 5, 4)
        OCR_LM(OCRDEC_Q4_0, 5, 4)
        OCR_LM(OCRDEC_U8A_G32, 5, 4)
    }
#undef OCR_LM
}

// Merge of the per-workgroup (best, index, second) partials: one workgroup
// per row, a strided pass then a tree in LDS (the merge is associative and
// commutative, so the result does not depend on the order).
//
// Status: a non-finite logit seen by any workgroup sets kStatLogit; a row
// without a finite winner (every logit NaN or -inf) gets token 0 and sets
// kStatNoToken.
__global__ __launch_bounds__(256) void argmax_final_kernel(const float* part, int n_wg, int rows, int32_t* tok_out,
                                                           float* top2, int32_t* gen_index, uint32_t* status) {
    __shared__ float sb[4], ss[4];
    __shared__ int si[4];
    const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // the generation index is requested with the partials (not after the merge)
    const int gi = (gen_index && tid == 0) ? gen_index[r] : 0;
    float b = -INFINITY, s = -INFINITY;
    int bi = 0x7fffffff;
    int fl = 0;
    for (int w = tid; w < n_wg; w += blockDim.x) {
        const float* e = part + ((int64_t)w * rows + r) * 4;
        argmax_merge(b, bi, s, e[0], __float_as_int(e[1]), e[2]);
        fl |= __float_as_int(e[3]);
    }
    fl = __syncthreads_or(fl);
    for (int o = 32; o > 0; o >>= 1) {
        const float b2 = __shfl_xor(b, o, 64), s2 = __shfl_xor(s, o, 64);
        const int i2 = __shfl_xor(bi, o, 64);
        argmax_merge(b, bi, s, b2, i2, s2);
    }
    if (lane == 0) {
        sb[wave] = b;
        ss[wave] = s;
        si[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) argmax_merge(b, bi, s, sb[w], si[w], ss[w]);
        if (tok_out) tok_out[r] = (bi == 0x7fffffff) ? 0 : bi;
        const uint32_t st = (uint32_t)(fl ? kStatLogit : 0) | (bi == 0x7fffffff ? kStatNoToken : 0);
        if (status && st) atomicOr(status, st);
        if (top2) {
            top2[2 * r] = b;
            top2[2 * r + 1] = s;
        }
        if (gen_index) gen_index[r] = gi + 1;
    }
}

void launch_argmax_final(const float* part, int n_wg, int rows, int32_t* tok_out, float* top2, int32_t* gen_index,
                         uint32_t* status, hipStream_t s) {
    hipLaunchKernelGGL(argmax_final_kernel, dim3(rows), dim3(256), 0, s, part, n_wg, rows, tok_out, top2, gen_index,
                       status);
}

}  // namespace ocrdec

using namespace ocrdec;

extern "C" ocrdec_status ocrdec_gemv_q(const ocrdec_qmat* W, int32_t rows, const uint16_t* x, int64_t ldx, void* y,
                                       int32_t y_type, int64_t ldy, void* stream) {
    ocrdec_status st = check_qmat(W, "W");
    if (st != OCRDEC_OK) return st;
    OCR_CHECK_ARG(rows >= 1 && rows <= 4096, "rows must be in [1, 4096]");
    OCR_CHECK_ARG(x && y, "x and y must be non-NULL");
    OCR_CHECK_ARG(ldx >= W->k && ldx % 8 == 0, "ldx must be >= k and a multiple of 8");
    OCR_CHECK_ARG(((uintptr_t)x & 15) == 0, "x must be 16-byte aligned");
    OCR_CHECK_ARG(ldy >= W->n, "ldy must be >= n");
    OCR_CHECK_ARG(y_type == OCRDEC_OUT_F32 || y_type == OCRDEC_OUT_F16, "unknown y_type");
    const int epi = y_type == OCRDEC_OUT_F32 ? EPI_F32 : EPI_F16;
    GemvPlan pl = plan_gemv(W->fmt, W->n, W->k, rows, epi);
    GemvParams p{};
    p.w = (const uint8_t*)W->data;
    p.n = W->n;
    p.k = W->k;
    p.nchunks = n_chunks(W->fmt, W->k);
    p.xs = XDirect{x, ldx, rows};
    p.y = y;
    p.ldy = ldy;
    launch_gemv(W->fmt, epi, pl, p, (hipStream_t)stream);
    return launch_status("ocrdec_gemv_q");
}

extern "C" ocrdec_status ocrdec_lm_argmax_workspace_bytes(const ocrdec_qmat* W, int32_t rows, size_t* bytes) {
    ocrdec_status st = check_qmat(W, "W");
    if (st != OCRDEC_OK) return st;
    OCR_CHECK_ARG(rows >= 1 && rows <= 32, "rows must be in [1, 32]");
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    *bytes = argmax_ws_bytes(plan_lm(W->fmt, W->n, W->k, rows).grid, rows);
    return OCRDEC_OK;
}

extern "C" ocrdec_status ocrdec_lm_argmax(const ocrdec_qmat* W, int32_t rows, const uint16_t* x, int32_t* tok_out,
                                          float* top2, void* ws, size_t ws_bytes, void* stream) {
    ocrdec_status st = check_qmat(W, "W");
    if (st != OCRDEC_OK) return st;
    OCR_CHECK_ARG(rows >= 1 && rows <= 32, "rows must be in [1, 32]");
    OCR_CHECK_ARG(x && tok_out, "x and tok_out must be non-NULL");
    OCR_CHECK_ARG(((uintptr_t)x & 15) == 0, "x must be 16-byte aligned");
    const LmPlan lp = plan_lm(W->fmt, W->n, W->k, rows);
    const size_t need = argmax_ws_bytes(lp.grid, rows);
    if (!ws || ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "argmax workspace: need " + std::to_string(need) + " bytes, got " +
                                              std::to_string(ws ? ws_bytes : 0));
    GemvParams p{};
    p.w = (const uint8_t*)W->data;
    p.n = W->n;
    p.k = W->k;
    p.nchunks = n_chunks(W->fmt, W->k);
    p.xs = XDirect{x, W->k, rows};
    p.part = (float*)ws;
    launch_lm_argmax(W->fmt, lp, p, (hipStream_t)stream);
    launch_argmax_final((float*)ws, lp.grid, rows, tok_out, top2, nullptr, nullptr, (hipStream_t)stream);
    return launch_status("ocrdec_lm_argmax");
}

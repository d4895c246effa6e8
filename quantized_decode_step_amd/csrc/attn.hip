// Single-query decode attention over a fixed prefix plus a ring of generated
// tokens ("Eseguire Unlimited-OCR su Apple Silicon con C e Metal", section "Il
// decoder e il Mixture of Experts": a 128-token ring keeps decode memory
// bounded), with an optional attention sink ("Nicolassuez/Falcon-OCR-int8-
// openvino": the sink is one more key whose value is zero, seeded at cache
// index 0).  The cache is caller-owned and only read, except for the new
// token's slot ("The KV cache is an INPUT").
//
// Split-KV: workgroup (split, head, row) scores up to 64 keys of the row's
// window, keeps them in LDS, and writes an unnormalised partial (max, sum,
// sum of p*v); a combine kernel merges the splits with the usual
// log-sum-exp rescaling.  (A last-arriving-workgroup merge inside the first
// kernel was measured slower twice: with device-scope fences, and with
// device-scope stores and an arrival counter, where waiting for the stores
// and then for the counter cost more than the second launch.  An online merge
// that requests every split's max, sum and output at once was slower too.)
// Keys are streamed with one 16-byte load per lane:
// for head_dim 128 a wavefront load covers 4 keys (16 lanes per key), for 64
// it covers 8 keys.
#include "attn.hpp"
#include "gemv_core.hpp"

#include <algorithm>
#include <cmath>

namespace ocrdec {

namespace {

constexpr int KPS = 64;  // keys per split

struct Window {
    int nkeys;     // keys attended
    int new_ord;   // ordinal of the new token in the window
    int new_idx;   // its cache index
    int pos;       // its RoPE position
    int P;         // prefix length
};

OCR_DEV Window row_window(const AttnParams& p, int r) {
    Window w;
    // Lengths are device data: clamp them so that no value can address memory
    // outside the row's cache (prefix <= prefix_cap in ring mode; room for the
    // new token in linear mode; t >= 0).
    const int pmax = p.ring_cap > 0 ? p.prefix_cap : p.prefix_cap - 1;
    w.P = min(max(p.prefix_len[r], 0), pmax);
    if (p.ring_cap > 0) {
        const int t = max(p.gen_index[r], 0);
        const int n_ring = min(t + 1, p.ring_cap);
        w.nkeys = w.P + n_ring;
        w.new_ord = w.P + t % p.ring_cap;
        w.new_idx = p.prefix_cap + t % p.ring_cap;
        w.pos = w.P + t;
    } else {
        w.nkeys = w.P + 1;
        w.new_ord = w.P;
        w.new_idx = w.P;
        w.pos = w.P - (p.sink ? 1 : 0);
    }
    return w;
}

OCR_DEV int ord_to_idx(const AttnParams& p, const Window& w, int o) {
    if (p.ring_cap > 0 && o >= w.P) return p.prefix_cap + (o - w.P);
    return o;
}

// RoPE (rotate-half) of lane pair (i, i + D/2) at position pos with
// frequency f = theta^(-2i/D) (computed on the host in double).  The angle
// pos * f is formed and reduced modulo 2*pi in double (positions reach
// thousands of radians), then rotated with a float sincos on [-pi, pi].
OCR_DEV void rope_pair(float x1, float x2, double f, int pos, float& y1, float& y2) {
    const double a = (double)pos * f;
    const double two_pi_hi = 6.283185307179586232, two_pi_lo = 2.4492935982947064e-16;
    const double n = rint(a * 0.15915494309189535);
    const double red = fma(-n, two_pi_lo, fma(-n, two_pi_hi, a));
    float sf, cf;
    sincosf((float)red, &sf, &cf);
    y1 = x1 * cf - x2 * sf;
    y2 = x2 * cf + x1 * sf;
}

}  // namespace

// INT8 KV cache (KV8): the cache holds int8 codes [rows][heads][cap][D] and
// one fp16 scale per (row, head, slot); the stored value is scale * code.
// The new token is quantised here: s = fp16(max|x| / 127) and code =
// round-half-away(x / s) clamped to +-127, both divisions correctly rounded
// in fp32; the attention reads the new token as stored, like every other key.
OCR_DEV void i8x16_to_f32(uint4 c, float (&v)[16]) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) v[4 * j + i] = (float)(int8_t)((w[j] >> (8 * i)) & 0xFF);
}

template <int D, bool KV8>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnParams p) {
    constexpr int VPL = KV8 ? 16 : 8;      // values per lane and key (one 16-byte load)
    constexpr int LPK = D / VPL;           // lanes per key
    constexpr int KPL = 64 / LPK;          // keys per wavefront load
    constexpr int ITER = KPS / (4 * KPL);  // key groups per wavefront
    __shared__ float q_s[D];
    __shared__ __align__(16) uint16_t knew_s[D];
    __shared__ __align__(16) uint16_t vnew_s[D];
    __shared__ __align__(16) int8_t knew8_s[KV8 ? D : 1];
    __shared__ __align__(16) int8_t vnew8_s[KV8 ? D : 1];
    __shared__ float snew_s[2];
    __shared__ float sc_s[KPS];
    __shared__ float o_s[4 * (64 / LPK)][D];  // p.V of every (wave, key group)
    __shared__ float red_s[8];

    const int s = blockIdx.x, h = blockIdx.y, r = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int HD = p.n_heads * D;
    // the projections do not depend on the window: request them first
    const float* qkv = p.qkv + (int64_t)r * p.ld_qkv;
    float xq1 = 0.f, xq2 = 0.f, xk1 = 0.f, xk2 = 0.f, xv = 0.f;
    if (tid < D / 2) {
        xq1 = qkv[h * D + tid];
        xq2 = qkv[h * D + tid + D / 2];
        xk1 = qkv[HD + h * D + tid];
        xk2 = qkv[HD + h * D + tid + D / 2];
    } else if (tid >= 64 && tid < 64 + D) {
        xv = qkv[2 * HD + h * D + tid - 64];
    }
    const int64_t head_off = ((int64_t)r * p.n_heads + h) * p.cache_cap;

    // ---- keys and values of this wavefront (wave w takes keys o0 + w*KPL +
    // it*4*KPL, one key per lane group), all requested before any use.  They
    // are requested before the window is known, at cache index = ordinal:
    // that is the key's slot whenever the prefix is full (and always in
    // linear mode), so the loads travel with the projections' instead of
    // waiting a round trip for the lengths.  Keys whose slot differs (ring
    // keys behind a shorter prefix) are requested again below; the new
    // token's slot is taken from LDS.
    const int dsub = (lane % LPK) * VPL;
    uint4 kr[ITER], vr[ITER];
    uint4 kr8[KV8 ? ITER : 1], vr8[KV8 ? ITER : 1];
    float ksc[KV8 ? ITER : 1], vsc[KV8 ? ITER : 1];
    auto load_kv = [&](int it, int ci) {
        if constexpr (KV8) {
            kr8[it] = *(const uint4*)((const int8_t*)p.k_cache + (head_off + ci) * D + dsub);
            vr8[it] = *(const uint4*)((const int8_t*)p.v_cache + (head_off + ci) * D + dsub);
            ksc[it] = h2f(p.k_scale[head_off + ci]);
            vsc[it] = h2f(p.v_scale[head_off + ci]);
        } else {
            kr[it] = *(const uint4*)(p.k_cache + (head_off + ci) * D + dsub);
            vr[it] = *(const uint4*)(p.v_cache + (head_off + ci) * D + dsub);
        }
    };
    {
        const int os0 = s * KPS, os1 = min(os0 + KPS, p.cache_cap);
#pragma unroll
        for (int it = 0; it < ITER; ++it) {
            const int o = os0 + wave * KPL + it * 4 * KPL + lane / LPK;
            if constexpr (KV8) {
                kr8[it] = vr8[it] = make_uint4(0, 0, 0, 0);
                ksc[it] = vsc[it] = 0.f;
            } else {
                kr[it] = vr[it] = make_uint4(0, 0, 0, 0);
            }
            if (o < os1) load_kv(it, o);
        }
    }
    const Window w = row_window(p, r);
    const int o0 = s * KPS, o1 = min(o0 + KPS, w.nkeys);
    float* part = p.part + (((int64_t)r * p.n_heads + h) * p.n_split + s) * (D + 2);
    if (o0 >= o1) return;  // beyond this row's window: not counted below
    const bool has_new = (w.new_ord >= o0 && w.new_ord < o1);
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int o = o0 + wave * KPL + it * 4 * KPL + lane / LPK;
        if (o < o1) {
            const int ci = ord_to_idx(p, w, o);
            if (ci != o) load_kv(it, ci);
        }
    }
    if (tid < D / 2) {
        const int i = tid;
        float y1, y2;
        rope_pair(xq1, xq2, p.inv_freq[i], w.pos, y1, y2);
        q_s[i] = h2f(f2h(y1));
        q_s[i + D / 2] = h2f(f2h(y2));
        if (has_new) {
            float k1, k2;
            rope_pair(xk1, xk2, p.inv_freq[i], w.pos, k1, k2);
            knew_s[i] = f2h(k1);
            knew_s[i + D / 2] = f2h(k2);
        }
    } else if (has_new && tid >= 64 && tid < 64 + D) {
        vnew_s[tid - 64] = f2h(xv);
    }
    __syncthreads();
    // the new token's codes (KV8, waves 0 and 1), stored to the cache at the end
    int8_t q8keep[KV8 ? D / 64 : 1];
    uint16_t s16keep = 0;
    if constexpr (KV8) {
        // wave 0 quantises the new key, wave 1 the new value (D / 64 values per lane)
        if (has_new && wave < 2) {
            constexpr int PER = D / 64;
            const uint16_t* src = wave == 0 ? knew_s : vnew_s;
            float x[PER], am = 0.f;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                x[j] = h2f(src[lane * PER + j]);
                am = fmaxf(am, fabsf(x[j]));
            }
            am = wave_max(am);
            const uint16_t s16 = f2h(__fdiv_rn(am, 127.0f));
            const float sf = h2f(s16);
            int8_t* dst = wave == 0 ? knew8_s : vnew8_s;
#pragma unroll
            for (int j = 0; j < PER; ++j) {
                const float qv = sf > 0.f ? fminf(fmaxf(roundf(__fdiv_rn(x[j], sf)), -127.f), 127.f) : 0.f;
                dst[lane * PER + j] = (int8_t)qv;
                q8keep[j] = (int8_t)qv;
            }
            s16keep = s16;
            if (lane == 0) snew_s[wave] = sf;
        }
        __syncthreads();
    }

    // ---- scores
    float qf[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) qf[i] = q_s[dsub + i];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int o = o0 + wave * KPL + it * 4 * KPL + lane / LPK;
        float dot = 0.f;
        if (o < o1) {
            const int ci = ord_to_idx(p, w, o);
            if constexpr (KV8) {
                const bool nw = ci == w.new_idx;
                float kf[16];
                i8x16_to_f32(nw ? *(const uint4*)(knew8_s + dsub) : kr8[it], kf);
#pragma unroll
                for (int i = 0; i < 16; ++i) dot = fmaf(qf[i], kf[i], dot);
                dot *= nw ? snew_s[0] : ksc[it];
            } else {
                const uint4 kv = ci == w.new_idx ? *(const uint4*)(knew_s + dsub) : kr[it];
                half8v kh = bits_to_half8(kv);
#pragma unroll
                for (int i = 0; i < 8; ++i) dot = fmaf(qf[i], (float)kh[i], dot);
            }
        }
        dot = group_sum<LPK>(dot);  // the key's LPK lanes
        if (o < o1 && (lane % LPK) == 0) {
            float sc = dot * p.scale;
            if (p.sink && ord_to_idx(p, w, o) == 0) sc += p.sink[h];
            sc_s[o - o0] = sc;
        }
    }
    __syncthreads();
    const int nk = o1 - o0;
    // ---- max and sum over the split's scores (wave 0)
    if (wave == 0) {
        float m = lane < nk ? sc_s[lane] : -INFINITY;
        m = wave_max(m);
        float e = lane < nk ? __expf(sc_s[lane] - m) : 0.f;
        if (lane < nk) sc_s[lane] = e;
        float l = wave_sum(e);
        if (lane == 0) {
            red_s[0] = m;
            red_s[1] = l;
        }
    }
    __syncthreads();
    // ---- p . V over the same key assignment
    float acc[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) acc[i] = 0.f;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int o = o0 + wave * KPL + it * 4 * KPL + lane / LPK;
        if (o < o1) {
            const int ci = ord_to_idx(p, w, o);
            if constexpr (KV8) {
                const bool nw = ci == w.new_idx;
                float vf[16];
                i8x16_to_f32(nw ? *(const uint4*)(vnew8_s + dsub) : vr8[it], vf);
                const float pj = sc_s[o - o0] * (nw ? snew_s[1] : vsc[it]);
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[i] = fmaf(pj, vf[i], acc[i]);
            } else {
                const uint4 vv = ci == w.new_idx ? *(const uint4*)(vnew_s + dsub) : vr[it];
                half8v vh = bits_to_half8(vv);
                const float pj = sc_s[o - o0];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(pj, (float)vh[i], acc[i]);
            }
        }
    }
    // sum over the key groups of all wavefronts through LDS (independent
    // reads instead of chains of cross-lane permutes), in a fixed order
#pragma unroll
    for (int i = 0; i < VPL; ++i) o_s[wave * (64 / LPK) + lane / LPK][dsub + i] = acc[i];
    __syncthreads();
    if (tid < D) {
        float o = 0.f;
#pragma unroll
        for (int j = 0; j < 4 * (64 / LPK); ++j) o += o_s[j][tid];
        part[tid] = o;
    }
    // The new token into the cache, last: nothing in this kernel reads it from
    // there (its split takes it from LDS), and a store issued earlier would
    // make every later barrier wait for it.
    if constexpr (KV8) {
        if (has_new && wave < 2) {
            constexpr int PER = D / 64;
            int8_t* gdst = (int8_t*)(wave == 0 ? p.k_cache : p.v_cache) + (head_off + w.new_idx) * D;
#pragma unroll
            for (int j = 0; j < PER; ++j) gdst[lane * PER + j] = q8keep[j];
            if (lane == 0) (wave == 0 ? p.k_scale : p.v_scale)[head_off + w.new_idx] = s16keep;
        }
    } else if (has_new && tid < D) {
        p.k_cache[(head_off + w.new_idx) * D + tid] = knew_s[tid];
        p.v_cache[(head_off + w.new_idx) * D + tid] = vnew_s[tid];
    }
    if (tid == 0) {
        part[D] = red_s[0];
        part[D + 1] = red_s[1];
    }

}

// Merge of the splits of one (head, row).  Everything the merge reads is
// requested before the row's window is known (the partial buffer holds
// n_split splits whatever the window; splits beyond it are ignored): thread
// t's split max and sum, and its output lane of the first 24 splits.  The
// maxima go through LDS, then each thread (one per output lane) sums the
// rescaled partial outputs in split order.
template <int D>
__global__ __launch_bounds__(D) void attn_combine_kernel(AttnParams p) {
    constexpr int PRE = 24;
    __shared__ float f_s[1024 + 1];
    __shared__ float red[2];
    const int h = blockIdx.x, r = blockIdx.y, tid = threadIdx.x;
    const int ns = p.n_split;
    const float* part0 = p.part + ((int64_t)r * p.n_heads + h) * ns * (D + 2);
    const float mv = tid < ns ? part0[tid * (D + 2) + D] : -INFINITY;
    const float lv = tid < ns ? part0[tid * (D + 2) + D + 1] : 0.f;
    float ov[PRE];
#pragma unroll
    for (int j = 0; j < PRE; ++j) ov[j] = j < ns ? part0[j * (D + 2) + tid] : 0.f;
    const Window w = row_window(p, r);
    const int n_used = (w.nkeys + KPS - 1) / KPS;
    if (tid < n_used) f_s[tid] = mv;
    for (int i = tid + D; i < n_used; i += D) f_s[i] = part0[i * (D + 2) + D];
    __syncthreads();
    if (tid < 64) {
        float M = -INFINITY;
        for (int i = tid; i < n_used; i += 64) M = fmaxf(M, f_s[i]);
        M = wave_max(M);
        if (tid == 0) red[0] = M;
    }
    __syncthreads();
    const float M = red[0];
    float Lp = 0.f;
    if (tid < n_used) {
        const float f = __expf(mv - M);
        Lp = lv * f;
        f_s[tid] = f;
    }
    for (int i = tid + D; i < n_used; i += D) {
        const float f = __expf(f_s[i] - M);
        Lp = fmaf(part0[i * (D + 2) + D + 1], f, Lp);
        f_s[i] = f;
    }
    if (D == 64) {
        Lp = wave_sum(Lp);
        if (tid == 0) red[1] = Lp;
    } else {
        Lp = wave_sum(Lp);
        __shared__ float l2[2];
        if ((tid & 63) == 0) l2[tid >> 6] = Lp;
        __syncthreads();
        if (tid == 0) red[1] = l2[0] + l2[1];
    }
    __syncthreads();
    float o = 0.f;
#pragma unroll
    for (int j = 0; j < PRE; ++j)
        if (j < n_used) o = fmaf(ov[j], f_s[j], o);
    int i = PRE;
    for (; i + 4 <= n_used; i += 4) {
        const float a0 = part0[(i + 0) * (D + 2) + tid];
        const float a1 = part0[(i + 1) * (D + 2) + tid];
        const float a2 = part0[(i + 2) * (D + 2) + tid];
        const float a3 = part0[(i + 3) * (D + 2) + tid];
        o = fmaf(a0, f_s[i], o);
        o = fmaf(a1, f_s[i + 1], o);
        o = fmaf(a2, f_s[i + 2], o);
        o = fmaf(a3, f_s[i + 3], o);
    }
    for (; i < n_used; ++i) o = fmaf(part0[i * (D + 2) + tid], f_s[i], o);
    p.out[(int64_t)r * p.ld_out + h * D + tid] = f2h(o / red[1]);
}

// Decode of up to 24 rows with head_dim 128: the merge of each head's
// splits and that head's share of the O projection in one launch, in place
// of the merge kernel, a launch gap and the O projection's GEMV.  Workgroup
// (g, hd, z) takes rows 4z .. 4z+3: thread group rg (128 threads) merges
// head hd of row 4z + rg (as attn_combine_kernel: the partials requested
// before the window is known) into LDS; its eight wavefronts then multiply
// the merged rows with the head's D columns of W_o for the 16-row tiles
// 8g .. 8g+7 (one tile each; the weights were requested before the merge) and
// add the products into the fixed-point residual with atomic integer adds:
// the residual receives one addend per head in the order the workgroups
// finish, and the integer sum is the same in any order.  Rows in groups of
// four over the grid (rather than passes of four in one workgroup) keep every
// merge to one round of dependent loads; each group reads the head's W_o
// columns again, from cache.
template <int FMT>
__global__ __launch_bounds__(512) void attn_merge_o_kernel(AttnParams p, const uint8_t* wo, int n_out, int64_t nchunks,
                                                           fix_t* h, int64_t ldh, uint32_t* status) {
    constexpr int D = 128, PRE = 24, KC = 32 * Geom<FMT>::SB, CPH = D / KC;
    extern __shared__ __align__(16) uint16_t xl[];  // [rows][n_heads * D + 8] fp16: head hd's columns
    __shared__ float f_s[4][1024 + 1];
    __shared__ float red[4], l2[4][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = blockIdx.x, hd = blockIdx.y, rbase = 4 * blockIdx.z;
    const int nr = min(4, p.rows - rbase);  // rows of this workgroup (>= 1)
    const int rg = tid >> 7, t = tid & 127;
    const int ldl = p.n_heads * D + 8;
    // thread group rg merges row rbase + rg into LDS row rg
    auto merge_row = [&](int rr) {
        const bool act = rr < nr;
        const int r = act ? rbase + rr : rbase;
        const int ns = p.n_split;
        const float* part0 = p.part + ((int64_t)r * p.n_heads + hd) * ns * (D + 2);
        const float mv = (act && t < ns) ? part0[t * (D + 2) + D] : -INFINITY;
        const float lv = (act && t < ns) ? part0[t * (D + 2) + D + 1] : 0.f;
        float ov[PRE];
#pragma unroll
        for (int j = 0; j < PRE; ++j) ov[j] = (act && j < ns) ? part0[j * (D + 2) + t] : 0.f;
        const Window w = row_window(p, r);
        const int n_used = act ? (w.nkeys + KPS - 1) / KPS : 0;
        float* fs = f_s[rg];
        if (t < n_used) fs[t] = mv;
        for (int i = t + D; i < n_used; i += D) fs[i] = part0[i * (D + 2) + D];
        __syncthreads();
        if (t < 64) {
            float M = -INFINITY;
            for (int i = t; i < n_used; i += 64) M = fmaxf(M, fs[i]);
            M = wave_max(M);
            if (t == 0) red[rg] = M;
        }
        __syncthreads();
        const float M = red[rg];
        float Lp = 0.f;
        if (t < n_used) {
            const float f = __expf(mv - M);
            Lp = lv * f;
            fs[t] = f;
        }
        for (int i = t + D; i < n_used; i += D) {
            const float f = __expf(fs[i] - M);
            Lp = fmaf(part0[i * (D + 2) + D + 1], f, Lp);
            fs[i] = f;
        }
        Lp = wave_sum(Lp);
        if ((t & 63) == 0) l2[rg][t >> 6] = Lp;
        __syncthreads();
        float o = 0.f;
#pragma unroll
        for (int j = 0; j < PRE; ++j)
            if (j < n_used) o = fmaf(ov[j], fs[j], o);
        for (int i = PRE; i < n_used; ++i) o = fmaf(part0[i * (D + 2) + t], fs[i], o);
        if (act) xl[rr * ldl + hd * D + t] = f2h(o / (l2[rg][0] + l2[rg][1]));
    };
    auto merge = [&]() { merge_row(rg); };
    const int tile = g * 8 + wave;
    const bool on = tile * 16 < n_out;
    const uint8_t* tp[1] = {wo + (int64_t)(on ? tile : 0) * nchunks * Geom<FMT>::CB};
    const int c0 = hd * CPH, c1 = on ? c0 + CPH : c0;
    float4v acc[1][1] = {{float4v{0.f, 0.f, 0.f, 0.f}}};
    kloop_lds<FMT, 1, 1, decltype(merge), CPH>(tp, c0, c1, merge, xl, ldl, nr, p.n_heads * D / 32, lane, acc);
    if (!on) return;
    bool bad = false;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int tok = 4 * (lane >> 4) + v, row = tile * 16 + (lane & 15);
        if (tok < nr && row < n_out) fix_atomic_add(h + (int64_t)(rbase + tok) * ldh + row, acc[0][0][v], bad);
    }
    report_status(status, bad, kStatResidual);
}

bool attn_merge_o_ok(const AttnParams& p, int fmt, int n_out) {
    // up to 24 rows (600 workgroups of 512 threads at 24; with 32 rows the
    // grid needs a second round and the merge kernel + O GEMV is as fast)
    if (p.rows < 1 || p.rows > 24 || p.head_dim != 128 || n_out % 16 != 0) return false;
    return fmt == OCRDEC_F16 || fmt == OCRDEC_Q8_0 || fmt == OCRDEC_Q4_0 || fmt == OCRDEC_U8A_G32;
}

void launch_attn_merge_o(const AttnParams& p0, int fmt, const uint8_t* wo, int n_out, fix_t* h, int64_t ldh,
                         uint32_t* status, hipStream_t s) {
    AttnParams p = p0;
    p.n_split = attn_n_split(p.cache_cap);
    dim3 g1(p.n_split, p.n_heads, p.rows);
    prof_mark(s, OCRDEC_K_ATTN);
    if (p.k_scale) hipLaunchKernelGGL((attn_partial_kernel<128, true>), g1, dim3(256), 0, s, p);
    else hipLaunchKernelGGL((attn_partial_kernel<128, false>), g1, dim3(256), 0, s, p);
    prof_mark(s, OCRDEC_K_ATTN_MERGE_O);
    const int HD = p.n_heads * 128;
    const int64_t nch = n_chunks(fmt, HD);
    const size_t lds = (size_t)std::min(p.rows, 4) * (HD + 8) * 2;
    dim3 g2((n_out / 16 + 7) / 8, p.n_heads, (p.rows + 3) / 4);
#define OCR_MO(F_) \
    case F_: hipLaunchKernelGGL(attn_merge_o_kernel<F_>, g2, dim3(512), lds, s, p, wo, n_out, nch, h, ldh, status); break;
    switch (fmt) {
        OCR_MO(OCRDEC_F16)
        OCR_MO(OCRDEC_Q8_0)
        OCR_MO(OCRDEC_Q4_0)
        OCR_MO(OCRDEC_U8A_G32)
    }
#undef OCR_MO
}

int attn_n_split(int cache_cap) { return (cache_cap + KPS - 1) / KPS; }

size_t attn_part_bytes(int rows, int n_heads, int head_dim, int cache_cap) {
    return align256((size_t)rows * n_heads * attn_n_split(cache_cap) * (head_dim + 2) * sizeof(float));
}

size_t attn_ws_bytes(int rows, int n_heads, int head_dim, int cache_cap) {
    return attn_part_bytes(rows, n_heads, head_dim, cache_cap);
}

void attn_set_rope(AttnParams& p, float theta) {
    for (int i = 0; i < 64; ++i)
        p.inv_freq[i] = i < p.head_dim / 2 ? std::pow((double)theta, -2.0 * i / p.head_dim) : 0.0;
}

// ---------------------------------------------------------------------------
// Prompt pass (prefill): causal attention of P positions of one row
// ("HunyuanOCR 的 ncnn 移植" 3.2: prefill and incremental decoding use causal
// masks of different shapes, and the decode steps reuse every layer's cache).
//
// prefill_rope_kernel: RoPE of q and k at the linear positions 0..P-1 (the
// same rotation as the decode kernel), q kept in a scratch buffer, k and v
// written to cache indices 0..P-1.
//
// attn_prefill_kernel: flash-style.  A workgroup of four wavefronts owns 64
// queries of one head (16 per wavefront) and walks the key blocks of 64 up to
// its last query, online softmax.  Both products run on MFMA in transposed
// form: S^T = K Q^T (keys on the MFMA rows, the wavefront's queries on its
// columns) and O^T = V^T P^T, so that every value a lane holds belongs to
// one query and the softmax rescaling is a per-lane factor.  P^T is the
// score accumulators converted in place to two fp16 terms each (hi + lo,
// so the weights keep about 22 bits): the 32 keys of one
// contraction step are taken in the order the two 16-key score tiles hold
// them (lane group g: keys 4g..4g+3 of each tile), and V^T is read from LDS
// in that same key order.  K stays key-major in LDS; V is stored transposed
// while it is staged.  The next two key blocks are in flight in registers
// while the current one is used.  A workgroup takes at most four key blocks:
// the windows of later query blocks are split over several workgroups (so
// the longest window does not set the kernel's length), whose unnormalised
// partials attn_prefill_merge_kernel combines.
// ---------------------------------------------------------------------------

template <int D, bool KV8>
__global__ __launch_bounds__(64) void prefill_rope_kernel(PrefillAttnParams p) {
    const int at = blockIdx.x, h = blockIdx.y, i = threadIdx.x;
    const bool on = i < D / 2;  // lane i holds the pair (i, i + D/2)
    // the sequence of packed position `at` (sequences are packed in order)
    int s = 0;
    while (s + 1 < p.n_seq && at >= p.seq_off[s + 1]) ++s;
    const int pos = at - p.seq_off[s];
    const int64_t crow = ((int64_t)p.seq_row[s] * p.n_heads + h) * p.cache_cap;
    const int HD = p.n_heads * D;
    const float* r = p.qkv + (int64_t)at * p.ld_qkv;
    uint16_t k1 = 0, k2 = 0, v1 = 0, v2 = 0;  // fp16 key and value pair
    if (on) {
        float y1, y2;
        rope_pair(r[h * D + i], r[h * D + i + D / 2], p.inv_freq[i], pos, y1, y2);
        uint16_t* qo = p.q + (int64_t)at * HD + h * D;
        qo[i] = f2h(y1);
        qo[i + D / 2] = f2h(y2);
        rope_pair(r[HD + h * D + i], r[HD + h * D + i + D / 2], p.inv_freq[i], pos, y1, y2);
        k1 = f2h(y1);
        k2 = f2h(y2);
        v1 = f2h(r[2 * HD + h * D + i]);
        v2 = f2h(r[2 * HD + h * D + i + D / 2]);
    }
    if constexpr (!KV8) {
        if (on) {
            uint16_t* kc = p.k_cache + (crow + pos) * D;
            kc[i] = k1;
            kc[i + D / 2] = k2;
            uint16_t* vc = p.v_cache + (crow + pos) * D;
            vc[i] = v1;
            vc[i + D / 2] = v2;
        }
    } else {
        // INT8 cache: one scale per key row and per value row, as in decode
        const float kx1 = h2f(k1), kx2 = h2f(k2), vx1 = h2f(v1), vx2 = h2f(v2);
        const float ka = wave_max(fmaxf(fabsf(kx1), fabsf(kx2))), va = wave_max(fmaxf(fabsf(vx1), fabsf(vx2)));
        const uint16_t ks16 = f2h(__fdiv_rn(ka, 127.0f)), vs16 = f2h(__fdiv_rn(va, 127.0f));
        const float ksf = h2f(ks16), vsf = h2f(vs16);
        auto code = [](float x, float sc) {
            return (int8_t)(sc > 0.f ? fminf(fmaxf(roundf(__fdiv_rn(x, sc)), -127.f), 127.f) : 0.f);
        };
        if (on) {
            int8_t* kc = (int8_t*)p.k_cache + (crow + pos) * D;
            kc[i] = code(kx1, ksf);
            kc[i + D / 2] = code(kx2, ksf);
            int8_t* vc = (int8_t*)p.v_cache + (crow + pos) * D;
            vc[i] = code(vx1, vsf);
            vc[i + D / 2] = code(vx2, vsf);
        }
        if (i == 0) {
            p.k_scale[crow + pos] = ks16;
            p.v_scale[crow + pos] = vs16;
        }
    }
}

constexpr int PQB = 64;  // queries per workgroup (16 per wavefront)
constexpr int PKB = 64;  // keys per block
constexpr int PKC = 4;   // key blocks per workgroup: longer windows are split over workgroups
constexpr int PREC = 36; // floats per lane in a partial record: 32 outputs, max, sum (padded)

// INT8 caches (KV8): the codes are staged in LDS as fp16 (exact), the key
// scales multiply the score accumulators and the value scales the
// probabilities, so both products stay exact up to fp32 accumulation.
OCR_DEV uint4 i8x8_to_h8(uint2 c) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t src = j < 2 ? c.x : c.y;
        const int sh = 16 * (j & 1);
        const f16_t a = (f16_t)(float)(int8_t)((src >> sh) & 0xFF);
        const f16_t b = (f16_t)(float)(int8_t)((src >> (sh + 8)) & 0xFF);
        w[j] = (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int D, bool KV8>
__global__ __launch_bounds__(256) void attn_prefill_kernel(PrefillAttnParams p) {
    constexpr int KS = D / 32;                 // contraction steps of the score product
    constexpr int DT = D / 16;                 // 16-wide output tiles
    constexpr int KLD = D + 8;                 // K block row stride (halves)
    constexpr int VLD = PKB + 8;               // transposed V block row stride (halves)
    constexpr int NPC = PKB * D / 8 / 256;     // 16-byte pieces per thread per block, K and V each
    __shared__ __align__(16) uint16_t k_s[PKB * KLD];
    __shared__ __align__(16) uint16_t vt_s[D * VLD];
    __shared__ float ksc_s[KV8 ? PKB : 1], vsc_s[KV8 ? PKB : 1];
    // workgroup (query block qb, chunk c of its key blocks, head h, sequence
    // sq); query block qb needs key blocks 0..qb, taken PKC at a time
    const int nch = (int)gridDim.x / p.n_qb;  // chunk slots per query block
    const int sq = blockIdx.z, P = p.seq_len[sq], n_qb = (P + PQB - 1) / PQB;
    const int slot = (int)blockIdx.x / nch, c = (int)blockIdx.x % nch, h = blockIdx.y;
    if (slot >= n_qb) return;  // uniform: a shorter sequence
    const int qb = n_qb - 1 - slot;
    const int n_c = (qb + PKC) / PKC;
    if (c >= n_c) return;  // uniform: this query block has fewer chunks
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
    const int HD = p.n_heads * D;
    const int64_t at0 = p.seq_off[sq];  // packed position of the sequence's first token
    const int q0 = qb * PQB;
    const int qw = q0 + 16 * wave + c16;  // this lane's query (an MFMA column)
    const int kb0 = c * PKC, nkb = min(kb0 + PKC, qb + 1);
    const int64_t crow = ((int64_t)p.seq_row[sq] * p.n_heads + h) * p.cache_cap;
    const uint16_t* kbase = p.k_cache + crow * D;
    const uint16_t* vbase = p.v_cache + crow * D;

    // queries (B operand of S^T = K Q^T): step ks holds d = 32 ks + 8 g .. + 7
    half8v qf[KS];
    {
        const uint16_t* qp = p.q + (at0 + min(qw, P - 1)) * HD + h * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = bits_to_half8(*(const uint4*)(qp + 32 * ks));
    }
    // staging: thread t carries key row t % 64, column pieces t / 64 + 4 i;
    // keys past the prompt are zero (their scores are masked, and a zero
    // value keeps the masked products finite)
    uint4 kr0[NPC], vr0[NPC], kr1[NPC], vr1[NPC];
    float sc0 = 0.f, sc1 = 0.f;  // KV8: key (threads 0..63) or value (64..127) scale of the staged row
    auto load_blk = [&](int kb, uint4(&kr)[NPC], uint4(&vr)[NPC], float& sc) {
        const int key = kb * PKB + (tid & 63);
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int c = (tid >> 6) + 4 * i;
            kr[i] = vr[i] = make_uint4(0, 0, 0, 0);
            if (key < P) {
                if constexpr (KV8) {
                    kr[i] = i8x8_to_h8(*(const uint2*)((const int8_t*)p.k_cache + (crow + key) * D + 8 * c));
                    vr[i] = i8x8_to_h8(*(const uint2*)((const int8_t*)p.v_cache + (crow + key) * D + 8 * c));
                } else {
                    kr[i] = *(const uint4*)(kbase + (int64_t)key * D + 8 * c);
                    vr[i] = *(const uint4*)(vbase + (int64_t)key * D + 8 * c);
                }
            }
        }
        if constexpr (KV8) {
            sc = 0.f;
            if (tid < 128 && key < P) sc = h2f((tid < 64 ? p.k_scale : p.v_scale)[crow + key]);
        }
    };
    auto store_blk = [&](const uint4(&kr)[NPC], const uint4(&vr)[NPC], float sc) {
        const int r = tid & 63;
        if constexpr (KV8) {
            if (tid < 64) ksc_s[r] = sc;
            else if (tid < 128) vsc_s[r] = sc;
        }
#pragma unroll
        for (int i = 0; i < NPC; ++i) {
            const int c = (tid >> 6) + 4 * i;
            *(uint4*)(k_s + r * KLD + 8 * c) = kr[i];
            const uint32_t w4[4] = {vr[i].x, vr[i].y, vr[i].z, vr[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                vt_s[(8 * c + 2 * j) * VLD + r] = (uint16_t)(w4[j] & 0xFFFF);
                vt_s[(8 * c + 2 * j + 1) * VLD + r] = (uint16_t)(w4[j] >> 16);
            }
        }
    };

    float4v o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = float4v{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    // two key blocks in flight: block kb + 2 is requested into the registers
    // block kb has just left for LDS
    auto step = [&](int kb, uint4(&kr)[NPC], uint4(&vr)[NPC], float& sc) {
        __syncthreads();  // the previous block's LDS reads are done
        store_blk(kr, vr, sc);
        __syncthreads();
        if (kb + 2 < nkb) load_blk(kb + 2, kr, vr, sc);
        // scores of the 64 keys (4 tiles of 16) for this lane's query
        float s[4][4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
            float4v acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const half8v ka = bits_to_half8(*(const uint4*)(k_s + (kt * 16 + c16) * KLD + 32 * ks + 8 * g));
                acc = mfma16(ka, qf[ks], acc);
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int key = kb * PKB + kt * 16 + 4 * g + v;
                float sv = acc[v] * p.scale;
                if constexpr (KV8) sv *= ksc_s[kt * 16 + 4 * g + v];
                s[kt][v] = key <= qw ? sv : -INFINITY;
            }
        }
        // online softmax: the block maximum over the 16 values and the four
        // lane groups that share the query
        float mb = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v) mb = fmaxf(mb, s[kt][v]);
        mb = fmaxf(mb, __shfl_xor(mb, 16, 64));
        mb = fmaxf(mb, __shfl_xor(mb, 32, 64));
        const float m_new = fmaxf(m_run, mb);  // finite: key 0 is in every query's window
        const float alpha = __expf(m_run - m_new);
        // probabilities as two fp16 terms, hi + lo (hi = fp16(e), lo = fp16(e - hi)):
        // their products with V are exact, so the weights keep ~22 bits
        float ls = 0.f;
        half8v pb[2], pl[2];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float e = __expf(s[kt][v] - m_new);
                ls += e;
                float ev = e;
                if constexpr (KV8) ev *= vsc_s[kt * 16 + 4 * g + v];
                const f16_t hi = (f16_t)ev;
                pb[kt >> 1][(kt & 1) * 4 + v] = hi;
                pl[kt >> 1][(kt & 1) * 4 + v] = (f16_t)(ev - (float)hi);
            }
        ls += __shfl_xor(ls, 16, 64);
        ls += __shfl_xor(ls, 32, 64);
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            o[dt] *= alpha;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const uint16_t* vp = vt_s + (dt * 16 + c16) * VLD + 32 * kk + 4 * g;
                const uint2 lo = *(const uint2*)vp, hi = *(const uint2*)(vp + 16);
                const half8v va = bits_to_half8(make_uint4(lo.x, lo.y, hi.x, hi.y));
                o[dt] = mfma16(va, pb[kk], o[dt]);
                o[dt] = mfma16(va, pl[kk], o[dt]);
            }
        }
    };
    load_blk(kb0, kr0, vr0, sc0);
    if (kb0 + 1 < nkb) load_blk(kb0 + 1, kr1, vr1, sc1);
    for (int kb = kb0; kb < nkb; kb += 2) {
        step(kb, kr0, vr0, sc0);
        if (kb + 1 < nkb) step(kb + 1, kr1, vr1, sc1);
    }
    if (n_c > 1) {
        // one of several chunks: the unnormalised partial of every lane (its
        // 4 DT outputs, the running max and sum) for the merge kernel
        float* rec = p.part + (((((int64_t)sq * p.n_heads + h) * p.n_qb + qb) * nch + c) * 256 + tid) * PREC;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) *(float4*)(rec + 4 * dt) = make_float4(o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
        rec[32] = m_run;
        rec[33] = l_run;
        return;
    }
    if (qw < P) {
        const float inv = 1.0f / l_run;
        uint16_t* op = p.out + (at0 + qw) * p.ld_out + h * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const uint32_t lo = (uint32_t)f2h(o[dt][0] * inv) | ((uint32_t)f2h(o[dt][1] * inv) << 16);
            const uint32_t hi = (uint32_t)f2h(o[dt][2] * inv) | ((uint32_t)f2h(o[dt][3] * inv) << 16);
            *(uint2*)(op + dt * 16 + 4 * g) = make_uint2(lo, hi);
        }
    }
}

// Merge of the chunks of every query block that has more than one: lane
// (wave, l) of chunk c holds query q0 + 16 wave + l % 16; the chunks are
// combined in chunk order (log-sum-exp rescaling), so the result does not
// depend on which chunk finished first.
template <int D>
__global__ __launch_bounds__(256) void attn_prefill_merge_kernel(PrefillAttnParams p, int nch) {
    constexpr int DT = D / 16;
    const int qb = blockIdx.x, h = blockIdx.y, sq = blockIdx.z, P = p.seq_len[sq];
    const int n_c = (qb + PKC) / PKC;
    if (n_c <= 1 || qb * PQB >= P) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, c16 = lane & 15;
    const int qw = qb * PQB + 16 * wave + c16;
    if (qw >= P) return;
    const float* base = p.part + ((((int64_t)sq * p.n_heads + h) * p.n_qb + qb) * nch * 256 + tid) * PREC;
    float M = -INFINITY;
    for (int c = 0; c < n_c; ++c) M = fmaxf(M, base[(int64_t)c * 256 * PREC + 32]);
    float L = 0.f;
    float4 o[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int c = 0; c < n_c; ++c) {
        const float* rec = base + (int64_t)c * 256 * PREC;
        const float f = __expf(rec[32] - M);
        L = fmaf(rec[33], f, L);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const float4 v = *(const float4*)(rec + 4 * dt);
            o[dt] = make_float4(fmaf(v.x, f, o[dt].x), fmaf(v.y, f, o[dt].y), fmaf(v.z, f, o[dt].z), fmaf(v.w, f, o[dt].w));
        }
    }
    const float inv = 1.0f / L;
    uint16_t* op = p.out + ((int64_t)p.seq_off[sq] + qw) * p.ld_out + h * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        const uint32_t lo = (uint32_t)f2h(o[dt].x * inv) | ((uint32_t)f2h(o[dt].y * inv) << 16);
        const uint32_t hi = (uint32_t)f2h(o[dt].z * inv) | ((uint32_t)f2h(o[dt].w * inv) << 16);
        *(uint2*)(op + dt * 16 + 4 * g) = make_uint2(lo, hi);
    }
}

int prefill_chunks(int P) { return ((P + PQB - 1) / PQB + PKC - 1) / PKC; }

size_t prefill_attn_part_bytes(int n_seq, int max_len, int n_heads) {
    const int n_qb = (max_len + PQB - 1) / PQB;
    return align256((size_t)n_seq * n_heads * n_qb * prefill_chunks(max_len) * 256 * PREC * sizeof(float));
}

void prefill_set_rope(PrefillAttnParams& p, float theta) {
    for (int i = 0; i < 64; ++i)
        p.inv_freq[i] = i < p.head_dim / 2 ? std::pow((double)theta, -2.0 * i / p.head_dim) : 0.0;
}

void launch_attn_prefill(const PrefillAttnParams& p0, hipStream_t s) {
    PrefillAttnParams p = p0;
    int max_len = 1;
    for (int i = 0; i < p.n_seq; ++i) max_len = std::max(max_len, p.seq_len[i]);
    p.n_qb = (max_len + PQB - 1) / PQB;
    const int nch = prefill_chunks(max_len);
    const dim3 gr(p.P, p.n_heads), ga(p.n_qb * nch, p.n_heads, p.n_seq), gm(p.n_qb, p.n_heads, p.n_seq);
    const bool kv8 = p.k_scale != nullptr;
#define OCR_PF(D_, K_)                                                                                   \
    prof_mark(s, OCRDEC_K_OTHER);                                                                         \
    hipLaunchKernelGGL((prefill_rope_kernel<D_, K_>), gr, dim3(64), 0, s, p);                             \
    prof_mark(s, OCRDEC_K_OTHER);                                                                         \
    hipLaunchKernelGGL((attn_prefill_kernel<D_, K_>), ga, dim3(256), 0, s, p);                            \
    if (nch > 1) prof_mark(s, OCRDEC_K_OTHER);                                                            \
    if (nch > 1) hipLaunchKernelGGL(attn_prefill_merge_kernel<D_>, gm, dim3(256), 0, s, p, nch);
    if (p.head_dim == 128) {
        if (kv8) { OCR_PF(128, true) } else { OCR_PF(128, false) }
    } else {
        if (kv8) { OCR_PF(64, true) } else { OCR_PF(64, false) }
    }
#undef OCR_PF
}

void launch_attn(const AttnParams& p, hipStream_t s) {
    dim3 g1(p.n_split, p.n_heads, p.rows);
    dim3 g2(p.n_heads, p.rows);
    const bool kv8 = p.k_scale != nullptr;
    if (p.head_dim == 128) {
        prof_mark(s, OCRDEC_K_ATTN);
        if (kv8) hipLaunchKernelGGL((attn_partial_kernel<128, true>), g1, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((attn_partial_kernel<128, false>), g1, dim3(256), 0, s, p);
        prof_mark(s, OCRDEC_K_ATTN_MERGE);
        hipLaunchKernelGGL(attn_combine_kernel<128>, g2, dim3(128), 0, s, p);
    } else {
        prof_mark(s, OCRDEC_K_ATTN);
        if (kv8) hipLaunchKernelGGL((attn_partial_kernel<64, true>), g1, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((attn_partial_kernel<64, false>), g1, dim3(256), 0, s, p);
        prof_mark(s, OCRDEC_K_ATTN_MERGE);
        hipLaunchKernelGGL(attn_combine_kernel<64>, g2, dim3(64), 0, s, p);
    }
}

ocrdec_status check_attn(const ocrdec_attn_args* a) {
    OCR_CHECK_ARG(a, "args is NULL");
    OCR_CHECK_ARG(a->rows >= 1, "rows must be >= 1");
    OCR_CHECK_ARG(a->n_heads >= 1 && a->n_heads <= 64, "n_heads must be in [1, 64]");
    if (a->head_dim != 64 && a->head_dim != 128)
        return fail(OCRDEC_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    OCR_CHECK_ARG(a->qkv && a->k_cache && a->v_cache && a->prefix_len && a->out, "NULL pointer in args");
    OCR_CHECK_ARG(a->ring_cap == 0 || a->gen_index, "gen_index is NULL in ring mode");
    OCR_CHECK_ARG(a->ld_qkv >= 3LL * a->n_heads * a->head_dim, "ld_qkv too small");
    OCR_CHECK_ARG(a->ld_out >= (int64_t)a->n_heads * a->head_dim, "ld_out too small");
    OCR_CHECK_ARG(a->prefix_cap >= 0 && a->ring_cap >= 0 && a->prefix_cap + a->ring_cap >= 1,
                  "prefix_cap and ring_cap must be >= 0 with a non-empty cache");
    // the merge kernel holds one weight per 64-key split in LDS (1024 splits)
    OCR_CHECK_ARG((int64_t)a->prefix_cap + a->ring_cap <= 65536, "prefix_cap + ring_cap must be <= 65536");
    // rows are a grid dimension of the attention kernels
    OCR_CHECK_ARG(a->rows <= 65535, "rows must be <= 65535");
    OCR_CHECK_ARG(((uintptr_t)a->k_cache & 15) == 0 && ((uintptr_t)a->v_cache & 15) == 0,
                  "caches must be 16-byte aligned");
    OCR_CHECK_ARG((a->k_scale == nullptr) == (a->v_scale == nullptr),
                  "k_scale and v_scale must both be given (int8 cache) or both be NULL (fp16 cache)");
    OCR_CHECK_ARG(a->rope_theta > 0.f, "rope_theta must be positive");
    return OCRDEC_OK;
}

}  // namespace ocrdec

using namespace ocrdec;

extern "C" ocrdec_status ocrdec_attn_workspace_bytes(const ocrdec_attn_args* a, size_t* bytes) {
    ocrdec_status st = check_attn(a);
    if (st != OCRDEC_OK) return st;
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    *bytes = attn_ws_bytes(a->rows, a->n_heads, a->head_dim, a->prefix_cap + a->ring_cap);
    return OCRDEC_OK;
}

extern "C" ocrdec_status ocrdec_attn_decode(const ocrdec_attn_args* a, void* ws, size_t ws_bytes, void* stream) {
    ocrdec_status st = check_attn(a);
    if (st != OCRDEC_OK) return st;
    const int cap = a->prefix_cap + a->ring_cap;
    const size_t need = attn_ws_bytes(a->rows, a->n_heads, a->head_dim, cap);
    if (!ws || ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "attention workspace: need " + std::to_string(need) + " bytes, got " +
                                              std::to_string(ws ? ws_bytes : 0));
    AttnParams p{};
    p.rows = a->rows;
    p.n_heads = a->n_heads;
    p.head_dim = a->head_dim;
    p.qkv = a->qkv;
    p.ld_qkv = a->ld_qkv;
    p.k_cache = a->k_cache;
    p.v_cache = a->v_cache;
    p.prefix_cap = a->prefix_cap;
    p.ring_cap = a->ring_cap;
    p.cache_cap = cap;
    p.prefix_len = a->prefix_len;
    p.gen_index = a->gen_index;
    p.sink = a->sink;
    p.k_scale = a->k_scale;
    p.v_scale = a->v_scale;
    attn_set_rope(p, a->rope_theta);
    p.scale = a->scale;
    p.out = a->out;
    p.ld_out = a->ld_out;
    p.n_split = attn_n_split(cap);
    p.part = (float*)ws;
    launch_attn(p, (hipStream_t)stream);
    return launch_status("ocrdec_attn_decode");
}

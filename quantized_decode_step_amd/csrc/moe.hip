// DeepSeek-V2-style MoE ("Eseguire Unlimited-OCR su Apple Silicon con C e
// Metal", section "Il decoder e il Mixture of Experts": 64 routed experts,
// top-6 routing, 2 shared experts; the runtime computes the routing, groups
// the tokens per expert, runs the projections and recombines the results).
//
//   router GEMV (fp32 logits)
//   -> route_group: top-k per token, then a stable counting sort of the
//      (token, rank) pairs by expert and the list of active experts (routed
//      experts with at least one token, then the shared experts with all
//      tokens) — all on the device, no host read-back
//   -> grouped gate/up GEMV with the SwiGLU in the epilogue (fp16 a per slot)
//   -> grouped down GEMV (fp32 y per slot)
//   -> combine: shared outputs, then the routed ones weighted by rank order,
//      summed in fp32 and added to the residual with one fp16 rounding.
#include "moe.hpp"

namespace ocrdec {

// ---------------------------------------------------------------------------
// Routing and grouping (one workgroup of 1024 threads = 16 wavefronts)
// ---------------------------------------------------------------------------

// The end of row r's top-k in one wavefront, once lane k < K holds the k-th
// choice `own`: the experts used (forced ones if given) go to idx_out
// [rows][K], their renormalised weights (softmax over the used experts'
// logits) to p.w and w_out, and the captures.  logit(e): the row's logit of
// expert e (bias added separately if non-NULL).
template <class LOGIT>
OCR_DEV void topk_finish(const MoeParams& p, int r, int own, LOGIT logit, const float* bias, int* idx_out,
                         float* w_out) {
    const int lane = threadIdx.x & 63;
    const int E = p.n_experts, K = p.top_k;
    int use = own;
    const bool forced = p.forced && p.forced[(int64_t)r * K] >= 0;
    if (forced && lane < K) use = p.forced[(int64_t)r * K + lane];
    use = min(max(use, 0), E - 1);  // device data: keep every index in range
    float lk = -INFINITY;
    if (lane < K) lk = logit(use) + (bias ? bias[use] : 0.f);
    const float m = wave_max(lk);
    const float ex = lane < K ? __expf(lk - m) : 0.f;
    const float den = wave_sum(ex);
    if (lane < K) {
        const float w = ex / den;
        idx_out[r * K + lane] = use;
        p.w[(int64_t)r * K + lane] = w;
        if (w_out) w_out[r * K + lane] = w;
        if (p.cap_idx) p.cap_idx[(int64_t)r * K + lane] = own;
        if (p.cap_w) p.cap_w[(int64_t)r * K + lane] = w;
    }
}

// Top-k of the rows of `lg` ([rows][E], fp32, row stride ldl; global memory
// or LDS; `bias` [E] added if non-NULL), one wavefront per row: lane l holds
// experts l, l+64, ...; each of the K rounds takes the wave-wide maximum (a
// DPP reduction) and the lowest expert holding it (a ballot), so ties go to
// the lower index; a NaN logit counts as -inf and a taken expert drops out.
// Writes the experts used (forced ones if given) to idx_out [rows][K], their
// renormalised weights and the captures.  Row r's logits are row r - lr0 of lg.
OCR_DEV void topk_rows(const MoeParams& p, const float* lg, int ldl, const float* bias, int* idx_out, int r0 = 0,
                       int r1 = -1, int nsl = 1, int64_t lsl = 0, float* w_out = nullptr, int lr0 = 0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int E = p.n_experts, K = p.top_k;
    const float taken = __builtin_nanf("");
    if (r1 < 0) r1 = p.rows;
    for (int r = r0 + wave; r < r1; r += nw) {
        const float* l = lg + (int64_t)(r - lr0) * ldl;
        // logit e: the sum of the k-slices' partial products, in slice order
        auto logit = [&](int e) {
            float x = l[e];
            for (int z = 1; z < nsl; ++z) x += l[z * lsl + e];
            return x;
        };
        float v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            float x = -INFINITY;
            if (e < E) {
                x = logit(e) + (bias ? bias[e] : 0.f);
                if (!(x == x)) x = -INFINITY;
            }
            v[j] = e < E ? x : taken;
        }
        int own = 0;  // lane k < K keeps the k-th choice
        for (int k = 0; k < K; ++k) {
            const float m = wave_max(fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])));
            int e = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const unsigned long long b = __ballot(v[j] == m);
                if (b) {
                    e = 64 * j + __ffsll((long long)b) - 1;
                    break;
                }
            }
            if ((e & 63) == lane) v[e >> 6] = taken;
            if (lane == k) own = e;
        }
        topk_finish(p, r, own, logit, bias, idx_out, w_out);
    }
}

// Top-k of one row whose E <= 64 logits l (bias included) sit in LDS, by
// rank: expert e's rank is the number of experts before it in the order
// (logit descending, then index ascending; NaN as -inf), which is the order
// in which topk_rows' rounds take them, so the result is the same.  Every
// wave counts, for all experts at once (lane e), the experts of its own
// share of the row that come before; the partial counts meet in LDS (part_s:
// 64 * 16 + 64 ints, expert e's counts at 16 * e, read with four 16-byte loads)
// and wave 0 sums them in wave order, finds the K experts of rank < K and
// finishes as topk_rows.  Every thread of the workgroup must call it (it holds
// a barrier); at most 16 waves.
OCR_DEV void topk_one_row_ranked(const MoeParams& p, const float* l, int r, int* idx_out, float* w_out, int* part_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int E = p.n_experts, K = p.top_k;
    auto val = [&](int e) {
        const float x = l[e];
        return (x == x) ? x : -INFINITY;
    };
    const float ve = val(min(lane, E - 1));
    const int per = (E + nw - 1) / nw, j0 = wave * per, j1 = min(E, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) {
        const float vj = val(j);
        cnt += (vj > ve || (vj == ve && j < lane)) ? 1 : 0;
    }
    if (wave == 0)
        for (int w = nw; w < 16; ++w) part_s[16 * lane + w] = 0;
    part_s[16 * lane + wave] = cnt;
    __syncthreads();
    if (wave == 0) {
        int rank = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int4 c4 = *(const int4*)(part_s + 16 * lane + 4 * q);
            rank += c4.x + c4.y + c4.z + c4.w;
        }
        // lane k < K learns the expert of rank k (one writer per rank)
        int* sel_s = part_s + 64 * 16;
        if (lane < E && rank < K) sel_s[rank] = lane;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int own = lane < K ? sel_s[lane] : 0;
        topk_finish(p, r, own, [&](int e) { return l[e]; }, nullptr, idx_out, w_out);
    }
}

// Grouping of up to 256 (row, rank) pairs in LDS.  Every expert keeps a
// 256-bit mask of the pairs routed to it; a pair's place among its expert's
// pairs (stable: by row, then rank) is the popcount of the mask below it.
// Outputs: perm/inv, vrows[slot] = the row of every grouped slot (routed
// slots [0, NP), then shared expert s at NP + s*R + row) and the list of
// work entries virt[v] = (expert, first slot, token count <= 16): the shared
// experts' row blocks first (their work is the largest), then each routed
// expert's tokens in blocks of 16.  mask_s: LDS [E][4] u64,
// counts_s/offsets_s: LDS [E(+1)].
OCR_DEV void group_pairs_small(const MoeParams& p, const int* idx_s, unsigned long long* mask_s, int* counts_s,
                               int* offsets_s, const float* w_s) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = p.rows, E = p.n_experts, K = p.top_k, S = p.n_shared;
    const int NP = R * K;
    const int rb = (R + 15) / 16;  // row blocks of a shared expert
    for (int i = tid; i < 4 * E; i += blockDim.x) mask_s[i] = 0ull;
    __syncthreads();
    for (int pi = tid; pi < NP; pi += blockDim.x)
        atomicOr(&mask_s[idx_s[pi] * 4 + (pi >> 6)], 1ull << (pi & 63));
    __syncthreads();
    // counts, exclusive offsets and the work list: wave 0, four experts per lane
    // (the lane's 16 mask words are read at once: mask_s holds 4 * 256 words)
    if (wave == 0) {
        int cnt[4], tot = 0, nb = 0;
        unsigned long long mk[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) mk[i] = mask_s[16 * lane + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            cnt[j] = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) cnt[j] += __popcll(mk[4 * j + w]);
            if (e >= E) cnt[j] = 0;
            tot += cnt[j];
            nb += (cnt[j] + 15) >> 4;
        }
        int incl = tot, nbi = nb;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            const int tb = __shfl_up(nbi, o, 64);
            if (lane >= o) {
                incl += t;
                nbi += tb;
            }
        }
        int base = incl - tot, vb = S * rb + nbi - nb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            if (e < E) {
                counts_s[e] = cnt[j];
                offsets_s[e] = base;
                for (int b = 0; 16 * b < cnt[j]; ++b)
                    p.virt[vb++] = make_int4(e, base + 16 * b, min(16, cnt[j] - 16 * b), 0);
            }
            base += cnt[j];
        }
        for (int i = lane; i < S * rb; i += 64) {
            const int sx = i / rb, b = i % rb;
            p.virt[i] = make_int4(E + sx, NP + sx * R + 16 * b, min(16, R - 16 * b), 0);
        }
        if (lane == 63) {
            offsets_s[E] = incl;
            p.n_virt[0] = S * rb + nbi;
        }
    }
    __syncthreads();
    for (int pi = tid; pi < NP; pi += blockDim.x) {
        const int e = idx_s[pi], wd = pi >> 6;
        int t = __popcll(mask_s[e * 4 + wd] & ((1ull << (pi & 63)) - 1ull));
        for (int w = 0; w < wd; ++w) t += __popcll(mask_s[e * 4 + w]);
        const int pos = offsets_s[e] + t;
        p.perm[pos] = pi;
        p.inv[pi] = pos;
        p.vrows[pos] = pi / K;
        if (p.sw) p.sw[pos] = w_s[pi];
        if (p.cap_perm) p.cap_perm[pos] = pi;
    }
    for (int i = tid; i < S * R; i += blockDim.x) {
        p.vrows[NP + i] = i % R;
        if (p.sw) p.sw[NP + i] = 1.f;
    }
    if (p.cap_counts)
        for (int e = tid; e < E; e += blockDim.x) p.cap_counts[e] = counts_s[e];
    if (p.cap_offsets)
        for (int e = tid; e <= E; e += blockDim.x) p.cap_offsets[e] = offsets_s[e];
}

// The grouping of group_pairs_small for one row, in wavefront 0 alone: the
// row's top_k experts are distinct, so every routed expert gets one token
// and an expert's entry, slot and place in the work list is the rank of its
// id among the chosen ones.  Same outputs as group_pairs_small with rows = 1
// (shared experts' entries first, then the routed ones by expert id).
OCR_DEV void group_one_row(const MoeParams& p, const int* idx_s, const float* w_s) {
    const int lane = threadIdx.x & 63;
    const int E = p.n_experts, K = p.top_k, S = p.n_shared;
    const int e = lane < K ? idx_s[lane] : 0x7fffffff;
    // (a forced choice may repeat an expert: equal ids rank by choice, one
    // entry per token, which the expert kernels treat like one of two tokens)
    // Every lane reads the K choices from LDS (independent reads, no chain of
    // lane exchanges).
    int rank = 0;
#pragma unroll 8
    for (int j = 0; j < K; ++j) {
        const int ej = idx_s[j];
        rank += (ej < e || (ej == e && j < lane)) ? 1 : 0;
    }
    if (lane < K) {
        p.virt[S + rank] = make_int4(e, rank, 1, 0);
        p.perm[rank] = lane;
        p.inv[lane] = rank;
        p.vrows[rank] = 0;
        if (p.sw) p.sw[rank] = w_s[lane];
        if (p.cap_perm) p.cap_perm[rank] = lane;
    }
    if (lane < S) {
        p.virt[lane] = make_int4(E + lane, K + lane, 1, 0);
        p.vrows[K + lane] = 0;
        if (p.sw) p.sw[K + lane] = 1.f;
    }
    if (lane == 0) p.n_virt[0] = S + K;
    if (p.cap_counts || p.cap_offsets) {
        for (int x = lane; x <= E; x += 64) {
            int chosen = 0, below = 0;
            for (int j = 0; j < K; ++j) {
                const int ej = __shfl(e, j, 64);
                chosen += ej == x ? 1 : 0;
                below += ej < x ? 1 : 0;
            }
            if (p.cap_counts && x < E) p.cap_counts[x] = chosen;
            if (p.cap_offsets) p.cap_offsets[x] = below;
        }
    }
}

// Scratch of the grouping: LDS for decode-sized batches, the workspace
// otherwise (generic pointers serve both).
struct GroupScratch {
    const int* idx;  // [NP] expert of every (row, rank) pair
    int* rank;       // [NP]
    int* hist;       // [nchunk][E]
    int* counts;     // [E]
    int* offsets;    // [E + 1]
};

// Stable counting sort of the (row, rank) pairs by expert (any number of
// pairs; the scratch is in the workspace).
// Outputs: perm/inv, vrows[slot] = the row of every grouped slot (as in
// group_pairs_small) and the work list virt[v] = (expert, first slot, token
// count): the shared experts first, then every active routed expert.
OCR_DEV void group_pairs(const MoeParams& p, const GroupScratch& g) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
    const int R = p.rows, E = p.n_experts, K = p.top_k, S = p.n_shared;
    const int NP = R * K;

    // per 64-pair chunk: rank of each pair among the equal experts before it
    // in the chunk, and the chunk's histogram (one ballot per distinct expert)
    const int nchunk = (NP + 63) / 64;
    for (int c = wave; c < nchunk; c += nw) {
        for (int e = lane; e < E; e += 64) g.hist[(int64_t)c * E + e] = 0;
        const int pi = c * 64 + lane;
        const bool ok = pi < NP;
        const int e = ok ? g.idx[pi] : -1;
        unsigned long long todo = __ballot(ok);
        int rank = 0;
        while (todo) {
            const int leader = __ffsll((long long)todo) - 1;
            const int le = __shfl(e, leader, 64);
            const unsigned long long m = __ballot(ok && e == le);
            if (ok && e == le) rank = __popcll(m & ((1ull << lane) - 1ull));
            if (lane == leader) g.hist[(int64_t)c * E + le] = __popcll(m);
            todo &= ~m;
        }
        if (ok) g.rank[pi] = rank;
    }
    __syncthreads();

    // per expert: exclusive prefix of the chunk histograms, counts
    for (int e = tid; e < E; e += blockDim.x) {
        int run = 0;
        for (int c = 0; c < nchunk; ++c) {
            const int h = g.hist[(int64_t)c * E + e];
            g.hist[(int64_t)c * E + e] = run;
            run += h;
        }
        g.counts[e] = run;
    }
    __syncthreads();
    // exclusive scan of counts and the compact list of active experts (wave 0)
    if (wave == 0) {
        int base = 0, act = 0;
        for (int eb = 0; eb < E; eb += 64) {
            const int e = eb + lane;
            const int cnt = e < E ? g.counts[e] : 0;
            int incl = cnt, ai = cnt > 0 ? 1 : 0;
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_up(incl, o, 64);
                const int ta = __shfl_up(ai, o, 64);
                if (lane >= o) {
                    incl += t;
                    ai += ta;
                }
            }
            const int excl = base + incl - cnt;
            if (e < E) g.offsets[e] = excl;
            if (e < E && cnt > 0) p.virt[S + act + ai - 1] = make_int4(e, excl, cnt, 0);
            base += __shfl(incl, 63, 64);
            act += __shfl(ai, 63, 64);
        }
        if (lane == 0) {
            g.offsets[E] = base;
            for (int s = 0; s < S; ++s) p.virt[s] = make_int4(E + s, NP + s * R, R, 0);
            p.n_virt[0] = act + S;
        }
    }
    __syncthreads();

    // scatter: grouped position and row of every pair
    for (int pi = tid; pi < NP; pi += blockDim.x) {
        const int e = g.idx[pi];
        const int t = g.hist[(int64_t)(pi / 64) * E + e] + g.rank[pi];
        const int pos = g.offsets[e] + t;
        p.perm[pos] = pi;
        p.inv[pi] = pos;
        p.vrows[pos] = pi / K;
    }
    for (int i = tid; i < S * R; i += blockDim.x) p.vrows[NP + i] = i % R;
    __syncthreads();
    if (p.cap_counts)
        for (int e = tid; e < E; e += blockDim.x) p.cap_counts[e] = g.counts[e];
    if (p.cap_offsets)
        for (int e = tid; e <= E; e += blockDim.x) p.cap_offsets[e] = g.offsets[e];
    if (p.cap_perm)
        for (int i = tid; i < NP; i += blockDim.x) p.cap_perm[i] = p.perm[i];
}

// Routing of many rows: logits come from a separate router GEMV.
__global__ __launch_bounds__(1024) void route_group_kernel(MoeParams p) {
    topk_rows(p, p.logits, p.n_experts, p.bias, p.idx);
    __syncthreads();
    group_pairs(p, GroupScratch{p.idx, p.rank, p.hist, p.counts, p.offsets});
}

// Top-k of many rows (large batches): 16 rows per workgroup, one wavefront
// per row, logits from the router GEMM in global memory (the sum of its
// k-slices' partial products).
__global__ __launch_bounds__(1024) void topk_kernel(MoeParams p) {
    const int r0 = blockIdx.x * 16;
    topk_rows(p, p.logits, p.n_experts, p.bias, p.idx, r0, min(r0 + 16, p.rows), max(p.lslices, 1), p.lslice);
}

// Grouping of any number of pairs in one workgroup.  Wave w takes the
// contiguous pair range [w*NP/16, (w+1)*NP/16) in rounds of 64 (one pair per
// lane, up to 16 rounds' expert ids loaded at once): per round, every expert's
// 64-bit mask of the wave's lanes holding it (in the wave's own LDS table)
// gives each pair its place among the round's earlier pairs of that expert,
// added to the wave's running count of the expert.  A scan of the sixteen
// waves' counts then places every wave's pairs after the earlier waves', so a
// pair's slot follows pair order within its expert.  Work entries are blocks
// of up to `blk` tokens (shared experts first); vrows[slot] as in
// group_pairs_small.  LDS: masks and counts [16][E] (E <= 256: 48 KiB).
__global__ __launch_bounds__(1024) void group_large_kernel(MoeParams p, int blk) {
    __shared__ unsigned long long mask_s[16 * 256];
    __shared__ int wcnt_s[16 * 256];
    __shared__ int run_s[256], offsets_s[257];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = p.rows, E = p.n_experts, K = p.top_k, S = p.n_shared;
    const int NP = R * K;
    unsigned long long* mask = mask_s + wave * E;
    int* wcnt = wcnt_s + wave * E;
    for (int e = lane; e < E; e += 64) {
        mask[e] = 0ull;
        wcnt[e] = 0;
    }
    const int pw0 = (int)((int64_t)NP * wave / 16), pw1 = (int)((int64_t)NP * (wave + 1) / 16);
    const unsigned long long below = (1ull << lane) - 1ull;
    // rounds of this wave, in batches of 16 (expert ids loaded together); with
    // one batch (NP <= 16384) the ids and places stay in registers
    const bool one = NP <= 16 * 1024;
    int ev[16], rv[16];
    for (int b0 = pw0; b0 < pw1; b0 += 16 * 64) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int pi = b0 + 64 * c + lane;
            ev[c] = pi < pw1 ? p.idx[pi] : -1;
        }
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            if (b0 + 64 * c >= pw1) break;  // uniform
            const int e = ev[c];
            if (e >= 0) atomicOr(&mask[e], 1ull << lane);
            __builtin_amdgcn_wave_barrier();
            unsigned long long m = 0ull;
            int base = 0;
            if (e >= 0) {
                m = mask[e];
                base = wcnt[e];
            }
            __builtin_amdgcn_wave_barrier();
            rv[c] = base + __popcll(m & below);
            if (e >= 0 && (m & below) == 0ull) {  // the expert's first lane of the round
                wcnt[e] = base + __popcll(m);
                mask[e] = 0ull;
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (!one) {
#pragma unroll
            for (int c = 0; c < 16; ++c) {
                const int pi = b0 + 64 * c + lane;
                if (pi < pw1) p.rank[pi] = rv[c];
            }
        }
    }
    __syncthreads();
    // exclusive scan of the waves' counts per expert; totals into run_s
    for (int e = tid; e < E; e += 1024) {
        int acc = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int c = wcnt_s[w * E + e];
            wcnt_s[w * E + e] = acc;
            acc += c;
        }
        run_s[e] = acc;
    }
    __syncthreads();
    // offsets and the work list (wave 0, four experts per lane)
    if (wave == 0) {
        const int rb = (R + blk - 1) / blk;
        int cnt[4], tot = 0, nb = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            cnt[j] = e < E ? run_s[e] : 0;
            tot += cnt[j];
            nb += (cnt[j] + blk - 1) / blk;
        }
        int incl = tot, nbi = nb;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o, 64);
            const int tb = __shfl_up(nbi, o, 64);
            if (lane >= o) {
                incl += t;
                nbi += tb;
            }
        }
        int base = incl - tot, vb = S * rb + nbi - nb;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * lane + j;
            if (e < E) {
                offsets_s[e] = base;
                for (int b = 0; b * blk < cnt[j]; ++b)
                    p.virt[vb++] = make_int4(e, base + b * blk, min(blk, cnt[j] - b * blk), 0);
            }
            base += cnt[j];
        }
        for (int i = lane; i < S * rb; i += 64) {
            const int sx = i / rb, b = i % rb;
            p.virt[i] = make_int4(E + sx, NP + sx * R + b * blk, min(blk, R - b * blk), 0);
        }
        if (lane == 63) {
            offsets_s[E] = incl;
            p.n_virt[0] = S * rb + nbi;
        }
    }
    __syncthreads();
    auto place = [&](int pi, int e, int r) {
        const int pos = offsets_s[e] + wcnt_s[wave * E + e] + r;
        p.perm[pos] = pi;
        p.inv[pi] = pos;
        p.vrows[pos] = pi / K;
        if (p.cap_perm) p.cap_perm[pos] = pi;
    };
    if (one) {
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const int pi = pw0 + 64 * c + lane;
            if (pi < pw1) place(pi, ev[c], rv[c]);
        }
    } else {
        for (int pi = pw0 + lane; pi < pw1; pi += 64) place(pi, p.idx[pi], p.rank[pi]);
    }
    for (int i = tid; i < S * R; i += 1024) p.vrows[NP + i] = i % R;
    if (p.cap_counts)
        for (int e = tid; e < E; e += 1024) p.cap_counts[e] = run_s[e];
    if (p.cap_offsets)
        for (int e = tid; e <= E; e += 1024) p.cap_offsets[e] = offsets_s[e];
}

// ---------------------------------------------------------------------------
// Expert GEMM for large token counts (prefill-shaped batches)
//
// Work item: entry v (up to 128 tokens of one expert) x column group cg, one
// workgroup of four wavefronts, two per CU.  The activations move through LDS
// in stages of 128 columns (two stage buffers of 128 x 128 fp16, 64 KiB): the
// workgroup requests stage s+1 with buffer loads straight into LDS before it
// multiplies stage s, so staging takes no registers.  Within a 256-byte row
// the 16-byte pieces are stored at piece ^ (row % 16): the sixteen rows of
// one MFMA operand read fall on different banks without padding.  Every
// wavefront holds two weight tiles in registers (requested two stages
// ahead) and forms block jj+1's operands (LDS reads, dequantisation) while
// block jj's v_mfma_f32_16x16x32_f16 run over the entry's token groups (the
// group index innermost; groups past the token count are skipped).  The
// fp16 block scale is applied to each block's fp32 product (exact products,
// fp32 sums).  SwiGLU: wave w takes the gate tile 4*cg + w and its up tile
// and writes fp16 silu(gate) * up; otherwise wave w takes tiles 8*cg + 2w,
// +1 and writes fp32.  Entries are dealt round-robin to the XCDs (workgroup
// id mod 8) with all their column groups, so an entry's activations are read
// into one L2 and every XCD gets a like mix of full and part-filled entries.
// Formats F16, Q8_0, Q4_0; k a multiple of 128.
// ---------------------------------------------------------------------------

constexpr int EG_TM = 128;   // tokens per work entry
constexpr int EG_KS = 128;   // activation columns per LDS stage
constexpr int EG_NW = 4;     // wavefronts per workgroup (two workgroups per CU)
constexpr int EG_NBUF = 2;   // LDS stage buffers: stage s+1 in flight while s is multiplied
constexpr int EG_LDS = EG_NBUF * EG_TM * EG_KS * 2;
constexpr int EG_NDMA = EG_TM * EG_KS * 2 / 1024 / EG_NW;  // 1 KiB stage loads per wave and stage

template <int FMT, bool GLU>
__global__ __launch_bounds__(64 * EG_NW, 2) void expert_gemm_kernel(GroupedParams p, int n_cg) {
    constexpr int SB = Geom<FMT>::SB, CB = Geom<FMT>::CB, KC = 32 * SB;
    constexpr int CPS = EG_KS / KC;  // weight chunks per stage and tile
    constexpr int NG = EG_TM / 16;
    constexpr int PD = 2;                                        // weight prefetch distance (stages)
    constexpr int NWL = 2 * CPS * (FMT == OCRDEC_F16 ? 1 : 2);  // weight load instructions per stage
    constexpr int RW = EG_TM / EG_NW;                           // stage rows loaded per wave
    static_assert(RW % 16 == 0 && RW == 4 * EG_NDMA, "staging geometry");
    extern __shared__ __align__(16) uint16_t xs_dyn[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n_ent = p.dense_rows > 0 ? (p.dense_rows + EG_TM - 1) / EG_TM : p.n_virt[0];
    // one work item: entry v, column group cg
    auto item = [&](const int v, const int cg, const int z) {
        int e, off, cnt;
        if (p.dense_rows > 0) {
            e = 0;
            off = v * EG_TM;
            cnt = min(EG_TM, p.dense_rows - off);
        } else {
            const int4 ent = p.virt[v];
            e = ent.x;
            off = ent.y;
            cnt = ent.z;
        }
        if (cnt <= 0) return;
        const uint8_t* base = (e < p.n_experts) ? p.w_routed + (int64_t)e * p.expert_bytes
                                                : p.w_shared + (int64_t)(e - p.n_experts) * p.expert_bytes;
        int tile[2];
        bool tv[2];
        if constexpr (GLU) {
            tile[0] = cg * EG_NW + wave;
            tv[0] = tv[1] = tile[0] < p.out_tiles;
            tile[1] = tile[0] + p.out_tiles;
        } else {
            tile[0] = cg * 2 * EG_NW + 2 * wave;
            tile[1] = tile[0] + 1;
            tv[0] = tile[0] < p.out_tiles;
            tv[1] = tile[1] < p.out_tiles;
        }
        const uint8_t* tp[2];
        // k-slice z: stages [z * kst, min((z + 1) * kst, k / 128)) of the k range
        const int ns_all = p.k / EG_KS;
        const int kst = p.kslices > 1 ? (ns_all + p.kslices - 1) / p.kslices : ns_all;
        const int s0 = z * kst, ns = min(ns_all - s0, kst);
        if (ns <= 0) return;
#pragma unroll
        for (int t = 0; t < 2; ++t)
            tp[t] = base + (int64_t)(tv[t] ? tile[t] : 0) * p.nchunks * CB + (int64_t)s0 * CPS * CB;

        // staging: wave w fills rows RW*w .. RW*w + RW-1 (RW = 128 / waves), four
        // per load instruction; lane l of instruction i carries row
        // RW*w + 4i + l/16 into stored piece
        // l % 16, which holds column piece (l % 16) ^ (row % 16) of the stage.
        // Rows past the token count repeat the last token (never stored).
        // Buffer loads (MUBUF) into LDS: unlike the FLAT form they leave the
        // compiler's vmcnt tracking of the weight registers exact.  Byte offsets
        // are 32-bit (the host keeps the activation extent below 2 GiB).
        const __amdgpu_buffer_rsrc_t xrs = __builtin_amdgcn_make_buffer_rsrc((void*)p.x, 0, 0x7fffffff, 0x00020000);
        uint32_t voff[EG_NDMA];
#pragma unroll
        for (int i = 0; i < EG_NDMA; ++i) {
            const int rr = min(RW * wave + 4 * i + (lane >> 4), cnt - 1);
            const int64_t sr = (GLU && p.dense_rows == 0) ? p.vrows[off + rr] : off + rr;
            voff[i] = (uint32_t)(2 * (sr * p.ldx + 8 * ((lane & 15) ^ ((4 * i + (lane >> 4)) & 15))));
        }
        auto stage_load = [&](int s, int b) {
            uint16_t* dst = xs_dyn + b * (EG_TM * EG_KS) + wave * RW * EG_KS;
#pragma unroll
            for (int i = 0; i < EG_NDMA; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(xrs, (lds_void_t*)(dst + i * 4 * EG_KS), 16, voff[i], 2 * (s0 + s) * EG_KS,
                                                         0, 0);
        };
        // operand reads: lane l, block jj of a stage -> row l % 16 of the group,
        // column piece 4 jj + l / 16
        int aoff[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) aoff[jj] = (lane & 15) * EG_KS + 8 * ((4 * jj + (lane >> 4)) ^ (lane & 15));

        auto wload = [&](int s, WRegs(&w)[2][CPS]) {
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int c = 0; c < CPS; ++c) load_wchunk<FMT>(tp[t] + (int64_t)(s * CPS + c) * CB, lane, w[t][c]);
        };
        float4v acc[2][NG];
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int g = 0; g < NG; ++g) acc[t][g] = float4v{0.f, 0.f, 0.f, 0.f};
        const float4v zero = {0.f, 0.f, 0.f, 0.f};
        // Weight operands of one (tile, 32-column block): the codes q as fp16
        // (exact) and the block scale d, applied to the block's fp32 product
        // (Q8_0, Q4_0: exact products, fp32 sums); F16: the weights.
        struct BPk {
            half8v h;
            float d;
        };
        // The main loop, specialised on the token groups that hold tokens (in
        // pairs): a part-filled entry skips the empty groups' MFMAs and reads.
        auto run = [&](auto nga) {
            constexpr int NGA = decltype(nga)::value;
            auto deq = [&](const WRegs(&w)[2][CPS], int jj, BPk(&o)[2]) {
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    o[t].h = wfrag<FMT>(w[t][jj / SB], jj % SB);
                    o[t].d = wscale<FMT>(w[t][jj / SB], jj % SB);
                }
            };
            // one block of the active token groups; the group index runs innermost
            // so consecutive MFMAs write different accumulators
            auto mma = [&](const half8v(&a)[NGA], const BPk(&b)[2]) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int g = 0; g < NGA; ++g) {
                        if constexpr (FMT != OCRDEC_F16) {
                            const float4v m = mfma16(a[g], b[t].h, zero);
#pragma unroll
                            for (int q = 0; q < 4; ++q) acc[t][g][q] = fmaf(b[t].d, m[q], acc[t][g][q]);
                        } else {
                            acc[t][g] = mfma16(a[g], b[t].h, acc[t][g]);
                        }
                    }
            };
            auto lds_a = [&](const uint16_t* xb, int jj, half8v(&a)[NGA]) {
#pragma unroll
                for (int g = 0; g < NGA; ++g) a[g] = *(const half8v*)(xb + g * 16 * EG_KS + aoff[jj]);
            };
            // Step s: stage s sits in LDS buffer s % EG_NBUF, its weights in w (W(s),
            // requested PD steps earlier), the next stage's in wn.  Block jj+1's
            // operands (LDS reads, dequantisation) are formed while block jj's MFMAs
            // run; the last block forms block 0 of the next stage from wn, carried
            // into the next step in bc.  w is refilled with W(s+PD) once its last
            // block has been formed.
            BPk bc[2];
            auto step = [&](int s, WRegs(&w)[2][CPS], const WRegs(&wn)[2][CPS]) {
                // stage s complete in LDS; every wave is done with stage s-1's buffer.
                // A plain s_barrier: a workgroup fence here would also wait for the
                // next stage's loads.  Every LDS read of stage s-1 has been consumed
                // by an MFMA before this point, so none is outstanding.
                asm volatile("s_barrier" ::: "memory");
                stage_load(min(s + EG_NBUF - 1, ns - 1), (s + EG_NBUF - 1) % EG_NBUF);
                __builtin_amdgcn_sched_barrier(0);  // stage loads before the weight loads (vmcnt order)
                const uint16_t* xb = xs_dyn + (s % EG_NBUF) * (EG_TM * EG_KS);
                half8v ac[NGA];
                lds_a(xb, 0, ac);
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    half8v an[NGA];
                    BPk bn[2];
                    if (jj < 3) {
                        lds_a(xb, jj + 1, an);
                        deq(w, jj + 1, bn);
                        if (jj == 2) wload(min(s + PD, ns - 1), w);
                    } else {
                        deq(wn, 0, bn);
                    }
                    mma(ac, bc);
#pragma unroll
                    for (int g = 0; g < NGA; ++g) ac[g] = an[g];
#pragma unroll
                    for (int t = 0; t < 2; ++t) bc[t] = bn[t];
                }
                // stage s+1 has landed once only the loads issued after it remain:
                // the weight loads of the step that requested it and of the
                // EG_NBUF - 2 steps since, and those steps' stage loads
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<NWL + (EG_NBUF - 2) * (EG_NDMA + NWL)>();
            };
            static_assert(PD == 2 && PD + 2 >= EG_NBUF, "prologue and wait counts");
            WRegs wq[PD][2][CPS];
#pragma unroll
            for (int u = 0; u + 1 < EG_NBUF; ++u) stage_load(min(u, ns - 1), u);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < PD; ++u) wload(min(u, ns - 1), wq[u]);
            deq(wq[0], 0, bc);
            wait_vmcnt<(EG_NBUF - 2) * EG_NDMA + PD * NWL>();  // stage 0 (ahead of the weight loads)
            for (int s = 0; s < ns; s += PD) {
                step(s, wq[0], wq[1]);
                if (s + 1 < ns) step(s + 1, wq[1], wq[0]);
            }
        };
        const int ngp = (cnt + 31) >> 5;
        if (ngp >= 4) run(std::integral_constant<int, 8>{});
        else if (ngp == 3) run(std::integral_constant<int, 6>{});
        else if (ngp == 2) run(std::integral_constant<int, 4>{});
        else run(std::integral_constant<int, 2>{});
        // epilogue (MFMA D layout: lane l, register q -> token 16g + 4(l/16) + q, column l % 16)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int tok = g * 16 + 4 * (lane >> 4) + q;
                if (tok >= cnt) continue;
                const int64_t slot = off + tok;
                if constexpr (GLU) {
                    if (tv[0])
                        ((uint16_t*)p.y)[slot * p.ldy + tile[0] * 16 + (lane & 15)] =
                            f2h(silu(acc[0][g][q]) * acc[1][g][q]);
                } else {
#pragma unroll
                    for (int t = 0; t < 2; ++t)
                        if (tv[t]) ((float*)p.y)[z * p.ly_slice + slot * p.ldy + tile[t] * 16 + (lane & 15)] = acc[t][g][q];
                }
            }
    };
    // one work item per workgroup: entries dealt round-robin to the XCDs
    // (workgroup id mod 8), all column groups of an entry on one XCD
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3, nz = max(p.kslices, 1);
    const int v = xcd + 8 * (j / (n_cg * nz)), r = j % (n_cg * nz);
    if (v < n_ent) item(v, r % n_cg, r / n_cg);  // uniform per workgroup
}

// Routing of up to 32 rows in one workgroup (BIAS: the router has a bias).
// Router GEMV: wave w computes
// tile w % T over k-split w / T (T = E/16 tiles); its first router chunks are
// requested before anything else, then the MoE input is staged in LDS: either
// formed here, x = fp16(RMSNorm(h) * gamma) from the fp32 residual (also
// written out for the expert kernels), or copied from x.  The k-splits are
// summed in a fixed order in LDS; top-k reads the logits from LDS; the
// grouping works in LDS.  Dynamic LDS: rows * (H + 8) halves.
// MODE: ROUTE_ALL, all rows (<= 32) in the one workgroup, as above;
// ROUTE_ONE, a batch of one row (its grouping is a few lane operations of
// wave 0); ROUTE_ROW, one workgroup per row (row = workgroup id) forms that
// row's input, logits and choice and writes them to p.idx / p.w, with no
// grouping (the expert kernels of the expert-indexed decode MoE find their
// tokens from p.idx).  A single row's top-k (E <= 64) is taken by rank over
// all waves.
enum { ROUTE_ALL = 0, ROUTE_ONE = 1, ROUTE_ROW = 2 };
template <int FMT, int NV, bool BIAS, int XT, int MODE = ROUTE_ALL>
__global__ __launch_bounds__(1024) void route_fused_kernel(MoeParams p, const uint8_t* router, int H,
                                                            const uint16_t* x, int64_t ldx, const fix_t* h_in,
                                                            const uint16_t* norm_w, float eps, uint16_t* x_out) {
    constexpr int CB = Geom<FMT>::CB;
    extern __shared__ __align__(16) uint16_t xl_dyn[];
    __shared__ float4v red[XT * 16 * 64];  // k-split partials of one pass (XT x 16 tokens)
    __shared__ float lg_s[32 * 256];  // logits [32][E <= 256]
    __shared__ int use_s[256], counts_s[256], offsets_s[257];
    __shared__ float wsel_s[256];
    __shared__ unsigned long long mask_s[4 * 256];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = p.n_experts, T = E / 16;
    constexpr bool ROW = MODE == ROUTE_ROW;
    const int r0 = ROW ? (int)blockIdx.x : 0, R = MODE == ROUTE_ALL ? p.rows : 1;
    // The arguments the serial tail (top-k, grouping) reads are requested
    // now: a scalar-cache miss there stalls the only workgroup for a memory
    // round trip.
    asm volatile("" ::"s"(p.perm), "s"(p.virt), "s"(p.cap_perm));
    const int nks = 16 / T;
    const int tile = wave % T, ks = wave / T;
    const int64_t nch = n_chunks_dev<FMT>(H);
    const int cper = (int)((nch + nks - 1) / nks);
    const int c0 = (int)min((int64_t)ks * cper, nch);  // (a chunk index in range even when empty)
    const int c1 = ks < nks ? (int)min((int64_t)(c0 + cper), nch) : c0;
    const uint8_t* tp[1] = {router + (int64_t)tile * nch * CB};
    const int ldl = xlds_stride(H);
    int staged = 0;
    auto stage = [&]() {
        if (staged) return;
        staged = 1;
        if (norm_w) {
            // three groups per lane: the 16-wave workgroup has 128 registers per lane
            block_rmsnorm_fix<3>(h_in, norm_w, H, eps, r0, R, x_out, ldx, xl_dyn, ldl);
        } else {
            stage_x<4>(XDirect{x + (int64_t)r0 * ldx, ldx, R}, 0, R, H, xl_dyn, ldl);
        }
    };
    // XT = 2: 17-32 rows in one pass over the router weights
    for (int tok0 = 0; tok0 < R; tok0 += 16 * XT) {
        float4v acc[1][XT];
#pragma unroll
        for (int xt = 0; xt < XT; ++xt) acc[0][xt] = float4v{0.f, 0.f, 0.f, 0.f};
        if constexpr (MODE != ROUTE_ALL) {
            if (norm_w) {
                // one row: its residual slices are requested ahead of the router
                // weights (they arrive first, and the norm is ready when the
                // weights are); a one-row workgroup has the registers for one
                // more chunk in flight
                RowNormFix<3> rn;
                auto pre = [&]() { rn.issue(h_in, norm_w, H, r0); };
                auto fin = [&]() { rn.finish(H, eps, r0, x_out, ldx, xl_dyn); };
                kloop_lds<FMT, 1, XT, decltype(fin), 5, decltype(pre)>(tp, c0, c1, fin, xl_dyn, ldl, 1, H / 32, lane,
                                                                       acc, pre);
            } else {
                kloop_lds<FMT, 1, XT, decltype(stage), 5>(tp, c0, c1, stage, xl_dyn, ldl, 1, H / 32, lane, acc);
            }
        } else {
            kloop_lds<FMT, 1, XT, decltype(stage), 4>(tp, c0, c1, stage, xl_dyn + tok0 * ldl, ldl, R - tok0, H / 32,
                                                      lane, acc);
        }
#pragma unroll
        for (int xt = 0; xt < XT; ++xt) red[(xt * 16 + wave) * 64 + lane] = acc[0][xt];
        __syncthreads();
        if (wave < T) {
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) {
                float4v a = red[(xt * 16 + wave) * 64 + lane];
                for (int o = 1; o < nks; ++o) a += red[(xt * 16 + wave + o * T) * 64 + lane];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int tok = tok0 + 16 * xt + 4 * (lane >> 4) + v;
                    const int e = wave * 16 + (lane & 15);
                    // (no load without a bias: a conditional load here makes the
                    // wave wait for every store in flight, the normalised rows too)
                    if constexpr (BIAS) lg_s[tok * E + e] = a[v] + p.bias[e];
                    else lg_s[tok * E + e] = a[v];
                }
            }
        }
        __syncthreads();
    }
    // (the k-split partials in red are consumed: its LDS holds the rank counts)
    if (R == 1 && E <= 64) {
        if constexpr (ROW) topk_one_row_ranked(p, lg_s, r0, p.idx, nullptr, (int*)red);
        else topk_one_row_ranked(p, lg_s, 0, use_s, p.sw ? wsel_s : nullptr, (int*)red);
    } else {
        if constexpr (ROW) topk_rows(p, lg_s, E, nullptr, p.idx, r0, r0 + 1, 1, 0, nullptr, r0);
        else topk_rows(p, lg_s, E, nullptr, use_s, 0, -1, 1, 0, p.sw ? wsel_s : nullptr);
    }
    if constexpr (ROW) {
        return;
    } else {
        if (R == 1) {
            // wavefront 0 chose the row's experts and groups them itself
            if (wave == 0) group_one_row(p, use_s, wsel_s);
            return;
        }
        if constexpr (MODE == ROUTE_ALL) {
            __syncthreads();
            group_pairs_small(p, use_s, mask_s, counts_s, offsets_s, wsel_s);
        }
    }
}

// Dynamic LDS of route_fused_kernel.
inline size_t route_lds_bytes(int rows, int H) { return (size_t)rows * (H + 8) * 2; }

// ---------------------------------------------------------------------------
// Grouped expert GEMV
//
// Work item (virtual expert v, tile group g).  GLU mode: the gate tile g and
// the up tile g + d_ff/16 of expert v over the tokens routed to it, SwiGLU in
// the epilogue, fp16 a[slot][col].  DOWN mode: tile g of the down matrix over
// the expert's slots of a, fp32 y[slot][row].
// ---------------------------------------------------------------------------

// Expert-indexed decode MoE: the tokens of work entry v, found from the chosen
// experts pidx [rows][top_k] (pair i = r * top_k + j, rows * top_k <= 256).
// Entries: shared expert s, 16-token block b at v = s * nb16 + b; then the
// routed experts that hold at least one token, in expert order (the A-th of
// them at v = S * nb16 + A, its second block, if any, at S * nb16 + n_active
// + A).  Entries past those hold nothing.  A routed expert's tokens are its
// pairs in pair order (row, then rank: the order a stable grouping gives).
// Writes the entry's expert to e and LDS lists of its tokens (at most 16):
// row, slot of a (a routed pair's slot is its pair index, shared expert s's
// slot of row r is rows * top_k + s * rows + r) and, if w_s is non-NULL, the
// combine weight (pw[pair]; shared: 1).  Every wave computes the expert and
// count from the same ballots, so both are uniform over the workgroup; wave 0
// writes the lists.  Returns the count.
OCR_DEV int expert_entry(const GroupedParams& p, int v, int& e, int* row_s, int* slot_s, float* w_s) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int R = p.rows, K = p.top_k, NP = R * K, E = p.n_experts;
    const int sv = p.n_shared * p.nb16;
    if (v < sv) {
        const int s = v / p.nb16, b = v % p.nb16, cnt = max(0, min(16, R - 16 * b));
        e = E + s;
        if (wave == 0 && lane < cnt) {
            const int r = 16 * b + lane;
            row_s[lane] = r;
            slot_s[lane] = NP + s * R + r;
            if (w_s) w_s[lane] = 1.f;
        }
        return cnt;
    }
    int id[4];
    float wt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int i = min(64 * j + lane, NP - 1);
        id[j] = p.pidx[i];
        wt[j] = w_s ? p.pw[i] : 0.f;
    }
    // the active experts as an E-bit mask (E <= 256), OR-reduced over the wave
    unsigned long long act[4] = {0ull, 0ull, 0ull, 0ull};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const unsigned long long bit = 64 * j + lane < NP ? 1ull << (id[j] & 63) : 0ull;
#pragma unroll
        for (int w = 0; w < 4; ++w) act[w] |= (id[j] >> 6) == w ? bit : 0ull;
    }
    const int nwd = (E + 63) >> 6;
    int nact = 0;
    for (int w = 0; w < nwd; ++w) {  // uniform
        act[w] = wave_or(act[w]);
        nact += __popcll(act[w]);
    }
    const int u = v - sv;
    const int b = u < nact ? 0 : 1, a = u - b * nact;
    if (b >= p.nb16 || a >= nact) return 0;
    // the a-th set bit of the mask
    e = 0;
    int before = 0;
    for (int w = 0; w < nwd; ++w) {
        const int c = __popcll(act[w]);
        if (a < before + c) {
            const bool hit = ((act[w] >> lane) & 1ull) && __popcll(act[w] & ((1ull << lane) - 1ull)) == a - before;
            e = min(max(64 * w + __ffsll((long long)__ballot(hit)) - 1, 0), E - 1);  // (exactly one lane hits)
            break;
        }
        before += c;
    }
    int base = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bool m = 64 * j + lane < NP && id[j] == e;
        const unsigned long long bal = __ballot(m);
        const int t = base + __popcll(bal & ((1ull << lane) - 1ull)) - 16 * b;
        if (wave == 0 && m && t >= 0 && t < 16) {
            row_s[t] = (64 * j + lane) / K;
            slot_s[t] = 64 * j + lane;
            if (w_s) w_s[t] = wt[j];
        }
        base += __popcll(bal);
    }
    return max(0, min(16, base - 16 * b));
}

template <int FMT, int XT, int KS, bool GLU, bool LDSX, bool HADD = false, bool BYEXP = false>
__global__ __launch_bounds__(256, (GLU || !LDSX) ? 2 : 3) void grouped_kernel(GroupedParams p) {
    constexpr int CB = Geom<FMT>::CB;
    constexpr int NT = GLU ? 2 : 1;
    extern __shared__ __align__(16) uint16_t xl_dyn[];
    __shared__ float4v red[(KS > 1) ? 4 * NT * XT * 64 : 1];
    static_assert(!BYEXP || (XT == 1 && KS == 1), "expert-indexed entries: 16 tokens, one wave per item");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int item = blockIdx.x * (4 / KS) + wave / KS;
    const int ks = wave % KS;
    const int v = item / p.groups_per_expert;
    const int g = item % p.groups_per_expert;
    // expert-indexed entries: token lists in LDS (row, slot, weight)
    __shared__ int tr_s[BYEXP ? 16 : 1], ts_s[BYEXP ? 16 : 1];
    __shared__ float tw_s[BYEXP ? 16 : 1];
    bool valid;
    int e, off, cnt;
    if constexpr (BYEXP) {
        // every wave of the workgroup works on entry v (KS = 1, whole tile
        // groups per expert): the count is uniform
        cnt = expert_entry(p, v, e, tr_s, ts_s, HADD ? tw_s : nullptr);
        __syncthreads();
        if (cnt == 0) return;
        valid = true;
        off = 0;
    } else {
        // the list entry is read unconditionally (in bounds: v is clamped) so
        // that it travels with the count in one round trip
        const int vc = min(v, p.max_virt - 1);
        const int n_virt = p.n_virt[0];
        const int4 ent = p.virt[vc];
        valid = v < n_virt && v < p.max_virt;
        e = valid ? ent.x : 0;
        off = valid ? ent.y : 0;
        cnt = valid ? ent.z : 0;
    }
    const uint8_t* base = (e < p.n_experts) ? p.w_routed + (int64_t)e * p.expert_bytes
                                            : p.w_shared + (int64_t)(e - p.n_experts) * p.expert_bytes;
    const uint8_t* tile[NT];
    int tidx[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        tidx[i] = GLU ? (i == 0 ? g : g + p.half_tiles) : g;
        tile[i] = base + (int64_t)tidx[i] * p.nchunks * CB;
    }
    const int cper = (int)((p.nchunks + KS - 1) / KS);
    const int c0 = (int)min((int64_t)ks * cper, p.nchunks);  // (a chunk index in range even when empty)
    const int c1 = valid ? (int)min((int64_t)(c0 + cper), p.nchunks) : c0;
    const int nblk = p.k / 32;
    // residual-adding down projection: the rows and weights of this lane's
    // slots travel with the weights (they depend only on the entry)
    int hrow[HADD ? XT : 1][4];
    float swt[HADD ? XT : 1][4];
    if constexpr (HADD) {
        {
#pragma unroll
            for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    const int t_ = min(16 * xt + 4 * (lane >> 4) + vv, max(cnt - 1, 0));
                    if constexpr (BYEXP) {
                        hrow[xt][vv] = tr_s[t_];
                        swt[xt][vv] = tw_s[t_];
                    } else {
                        const int s_ = off + t_;
                        hrow[xt][vv] = p.one_row ? 0 : p.vrows[s_];
                        swt[xt][vv] = p.sw[s_];
                    }
                }
        }
    }
    // token passes: the workgroup loops to the largest count among its waves
    int passes = (cnt + 16 * XT - 1) / (16 * XT);
    for (int pass = 0;; ++pass) {
        // all waves of the workgroup run the same number of passes
        int my_more = pass < passes ? 1 : 0;
        if (!__syncthreads_or(my_more)) break;
        const int tok0 = pass * 16 * XT;
        float4v acc[NT][XT];
#pragma unroll
        for (int i = 0; i < NT; ++i)
#pragma unroll
            for (int xt = 0; xt < XT; ++xt) acc[i][xt] = float4v{0.f, 0.f, 0.f, 0.f};
        const int cc1 = my_more ? c1 : c0;
        if constexpr (LDSX) {
            // the workgroup's waves share one expert (groups_per_expert is a
            // multiple of the waves per workgroup), hence one token set
            const int ldl = xlds_stride(p.k);
            // the pass's token rows go into LDS by direct buffer loads issued
            // ahead of the weight ring (pre); stage() waits for all but the
            // ring's loads
            constexpr int PFL = kloop_lds_depth<FMT, NT>();
            auto pre = [&]() {
                stage_rows_direct(
                    [&](int t) {
                        int row;
                        if constexpr (GLU) row = BYEXP ? tr_s[tok0 + t] : p.vrows[off + tok0 + t];
                        else if constexpr (BYEXP) row = ts_s[tok0 + t];
                        else row = off + tok0 + t;
                        return p.x + (int64_t)__builtin_amdgcn_readfirstlane(row) * p.ldx;
                    },
                    min(16 * XT, cnt - tok0), p.k, xl_dyn, ldl);
            };
            auto stage = [&]() { wait_vmcnt<kloop_prologue_loads<FMT, NT, PFL>()>(); };
            kloop_lds<FMT, NT, XT, decltype(stage), PFL, decltype(pre)>(tile, c0, cc1, stage, xl_dyn, ldl, cnt - tok0,
                                                                       nblk, lane, acc, pre);
        } else if constexpr (GLU) {
            if (!BYEXP && p.one_row) {
                // every slot reads row 0: no row-list load before the activations
                XDirect xs{p.x, p.ldx, 1};
                kloop<FMT, NT, XT>(tile, c0, cc1, xs, tok0, nblk, lane, acc);
            } else {
                XGather xs{p.x, p.ldx, BYEXP ? tr_s : p.vrows + off, cnt};
                kloop<FMT, NT, XT>(tile, c0, cc1, xs, tok0, nblk, lane, acc);
            }
        } else if constexpr (BYEXP) {
            XGather xs{p.x, p.ldx, ts_s, cnt};
            kloop<FMT, NT, XT>(tile, c0, cc1, xs, tok0, nblk, lane, acc);
        } else {
            XDirect xs{p.x + (int64_t)off * p.ldx, p.ldx, cnt};
            kloop<FMT, NT, XT>(tile, c0, cc1, xs, tok0, nblk, lane, acc);
        }
        ksplit_reduce<NT, XT, KS>(acc, red, wave, lane);
        bool bad = false;
        if (ks == 0 && my_more) {
#pragma unroll
            for (int xt = 0; xt < XT; ++xt)
#pragma unroll
                for (int vv = 0; vv < 4; ++vv) {
                    const int tok = tok0 + 16 * xt + 4 * (lane >> 4) + vv;
                    if (tok >= cnt) continue;
                    const int64_t slot = BYEXP ? ts_s[tok] : off + tok;
                    if constexpr (GLU) {
                        const int col = tidx[0] * 16 + (lane & 15);
                        const float gv = acc[0][xt][vv], uv = acc[1][xt][vv];
                        ((uint16_t*)p.y)[slot * p.ldy + col] = f2h(silu(gv) * uv);
                    } else {
                        const int row = tidx[0] * 16 + (lane & 15);
                        float* yp = (float*)p.y + slot * p.ldy + row;
                        if constexpr (HADD) {
                            // one pass per entry here (entries of <= 16 tokens)
                            fix_atomic_add(p.h + (int64_t)hrow[xt][vv] * p.ldh + row, swt[xt][vv] * acc[0][xt][vv],
                                           bad);
                        } else {
                            *yp = acc[0][xt][vv];
                        }
                    }
                }
        }
        if constexpr (HADD) report_status(p.status, bad, kStatResidual);
        __syncthreads();
    }
}

// Streamed grouped expert GEMV for decode batches (work entries of at most
// 16 tokens, activations staged in LDS).  A workgroup of four waves owns
// 4 * IPW consecutive work items of one entry (GLU: gate/up tile pairs; down:
// output tiles), so the waves share one staging of the entry's token rows.
// Each wave streams its IPW items as one sequence of (item, chunk) through a
// register ring of PF chunks that runs on from one item into the next, so the
// weight stream does not drain between items and a workgroup's start-up
// (work-list read, staging) is paid once for IPW items.  Epilogues as in
// grouped_kernel (SwiGLU into a; down: y, or weight x output added into the
// fixed-point residual).
template <int FMT, bool GLU, bool HADD, int IPW, int PF, bool BYEXP = false>
__global__ __launch_bounds__(256, 2) void grouped_stream_kernel(GroupedParams p) {
    constexpr int CB = Geom<FMT>::CB, SB = Geom<FMT>::SB;
    constexpr int NT = GLU ? 2 : 1;
    extern __shared__ __align__(16) uint16_t xl_dyn[];
    // (the wave index read as a scalar: chunk addresses are then scalar bases
    // plus the lane's fixed offset, with no per-lane 64-bit address math)
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wpe = p.groups_per_expert / (4 * IPW);  // workgroups per entry
    const int v = blockIdx.x / wpe;
    const int g0 = (blockIdx.x % wpe) * 4 * IPW + wave * IPW;
    __shared__ int tr_s[BYEXP ? 16 : 1], ts_s[BYEXP ? 16 : 1];
    __shared__ float tw_s[BYEXP ? 16 : 1];
    int e, off, cnt;
    if constexpr (BYEXP) {
        cnt = expert_entry(p, v, e, tr_s, ts_s, HADD ? tw_s : nullptr);
        __syncthreads();
        if (cnt == 0) return;  // uniform over the workgroup
        off = 0;
    } else {
        const int vc = min(v, p.max_virt - 1);
        const int n_virt = p.n_virt[0];
        const int4 ent = p.virt[vc];
        if (!(v < n_virt && v < p.max_virt)) return;  // uniform over the workgroup
        e = ent.x;
        off = ent.y;
        cnt = min(ent.z, 16);
    }
    e = __builtin_amdgcn_readfirstlane(e);  // (uniform: weight addresses stay scalar)
    const uint8_t* base = (e < p.n_experts) ? p.w_routed + (int64_t)e * p.expert_bytes
                                            : p.w_shared + (int64_t)(e - p.n_experts) * p.expert_bytes;
    const int nc = (int)p.nchunks;
    const int total = IPW * nc;
    auto tile_of = [&](int i, int t) { return (GLU && t == 1) ? g0 + i + p.half_tiles : g0 + i; };
    const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc((void*)base, 0, 0x7fffffff, 0x00020000);
    auto chunk_off = [&](int q, int t) {  // byte offset of the wave's chunk q of tile stream t
        const int qc = min(q, total - 1);
        return (uint32_t)(tile_of(qc / nc, t) * nc + (qc % nc)) * (uint32_t)CB;
    };
    // residual-adding down projection: rows and weights of this lane's slots
    int hrow[4];
    float swt[4];
    if constexpr (HADD) {
#pragma unroll
        for (int vv = 0; vv < 4; ++vv) {
            const int t_ = min(4 * (lane >> 4) + vv, max(cnt - 1, 0));
            if constexpr (BYEXP) {
                hrow[vv] = tr_s[t_];
                swt[vv] = tw_s[t_];
            } else {
                hrow[vv] = p.one_row ? 0 : p.vrows[off + t_];
                swt[vv] = p.sw[off + t_];
            }
        }
    }
    // The entry's token rows go into LDS by buffer loads that write LDS
    // directly (wave w copies rows w, w+4, ...; one instruction per 64 pieces
    // of 16 bytes of a row), issued ahead of the weight ring: loads return in
    // issue order, so the rows are in once all but the ring's loads are.
    const int ldl = xlds_stride(p.k);
    stage_rows_direct(
        [&](int t) {
            int row;
            if constexpr (GLU) row = BYEXP ? tr_s[t] : p.vrows[off + t];
            else if constexpr (BYEXP) row = ts_s[t];
            else row = off + t;
            return p.x + (int64_t)__builtin_amdgcn_readfirstlane(row) * p.ldx;
        },
        cnt, p.k, xl_dyn, ldl);
    __builtin_amdgcn_sched_barrier(0);
    WRegs wb[PF][NT];
#pragma unroll
    for (int u = 0; u < PF; ++u)
#pragma unroll
        for (int t = 0; t < NT; ++t) load_wchunk_rs<FMT>(wrs, chunk_off(u, t), lane, wb[u][t]);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<PF * NT * (FMT == OCRDEC_F16 ? 1 : 2)>();  // everything but the ring: the rows are in LDS
    __syncthreads();
    float* btab = (float*)(xl_dyn + 16 * ldl);  // Q4_0: the blocks' accumulator inputs, after the rows
    if constexpr (FMT == OCRDEC_Q4_0) {
        q4_split_prepare(xl_dyn, ldl, cnt, p.k / 32, p.k / 32, btab);
        __syncthreads();
    }
    float4v acc[NT][1];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][0] = float4v{0.f, 0.f, 0.f, 0.f};
    bool bad = false;
    // (PF divides the stream's length, checked by the host: every pass of the
    // ring is whole and the refills are unconditional, past the end they
    // repeat the last chunk, from cache; with no branch around them the
    // ring's registers stay in place across the loop's back edge)
    for (int q0 = 0; q0 < total; q0 += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int q = q0 + u;
            {
                const int c = q % nc;
                half8v xa[SB][1];
                float4v xs[SB][1];
                lds_xfrags_all<FMT>(xl_dyn, ldl, c, lane, xa);
                if constexpr (FMT == OCRDEC_Q4_0) {
                    float4v nb[4][1];
#pragma unroll
                    for (int j = 0; j < 4; ++j) nb[j][0] = *(const float4v*)(btab + 16 * (4 * c + j) + 4 * (lane >> 4));
                    chunk_mac_q4b<NT, 1, true>(wb[u], xa, nb, acc);
                } else {
                    xsums<FMT, 1>(xa, xs);
                    chunk_mac_tiles<FMT, NT>(wb[u], xa, xs, acc);
                }
#pragma unroll
                for (int t = 0; t < NT; ++t) load_wchunk_rs<FMT>(wrs, chunk_off(q + PF, t), lane, wb[u][t]);
                if (c == nc - 1) {  // item q / nc complete
                    const int i = q / nc;
                    if constexpr (FMT == OCRDEC_Q4_0) scale_acc<NT, 1>(acc, Q4_RAW_SCALE);  // (raw codes)
#pragma unroll
                    for (int vv = 0; vv < 4; ++vv) {
                        const int tok = 4 * (lane >> 4) + vv;
                        if (tok >= cnt) continue;
                        const int64_t slot = BYEXP ? ts_s[tok] : off + tok;
                        if constexpr (GLU) {
                            const int col = tile_of(i, 0) * 16 + (lane & 15);
                            ((uint16_t*)p.y)[slot * p.ldy + col] = f2h(silu(acc[0][0][vv]) * acc[1][0][vv]);
                        } else {
                            const int row = tile_of(i, 0) * 16 + (lane & 15);
                            if constexpr (HADD)
                                fix_atomic_add(p.h + (int64_t)hrow[vv] * p.ldh + row, swt[vv] * acc[0][0][vv], bad);
                            else ((float*)p.y)[slot * p.ldy + row] = acc[0][0][vv];
                        }
                    }
#pragma unroll
                    for (int t = 0; t < NT; ++t) acc[t][0] = float4v{0.f, 0.f, 0.f, 0.f};
                }
            }
        }
    }
    if constexpr (HADD) report_status(p.status, bad, kStatResidual);
}

// x = fp16(RMSNorm(h) * gamma) of one fixed-point residual row per workgroup.
__global__ __launch_bounds__(256) void moe_norm_kernel(const fix_t* h, const uint16_t* gamma, int H, float eps,
                                                       uint16_t* x, int64_t ldx) {
    __shared__ float red[4];
    const int r = blockIdx.x, tid = threadIdx.x;
    const fix_t* hr = h + (int64_t)r * H;
    float ss = 0.f;
    for (int c = tid; c < H; c += blockDim.x) ss = fmaf(fix_to(hr[c]), fix_to(hr[c]), ss);
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
    for (int c = tid; c < H; c += blockDim.x) x[(int64_t)r * ldx + c] = f2h(fix_to(hr[c]) * inv * h2f(gamma[c]));
}

// ---------------------------------------------------------------------------
// Combine (+ optional RMSNorm of the updated residual): one workgroup per row
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void combine_kernel(CombineParams p) {
    __shared__ float red[16];
    __shared__ float w_s[8];
    __shared__ int slot_s[16];
    const int r = blockIdx.x, tid = threadIdx.x;
    const int K = p.top_k, R = p.rows, H = p.hidden, S = p.n_shared;
    if (tid < K) {
        w_s[tid] = p.w[r * K + tid];
        slot_s[tid] = p.inv[r * K + tid];
    } else if (tid >= 64 && tid < 64 + S) {
        slot_s[8 + tid - 64] = p.np + (tid - 64) * R + r;
    }
    __syncthreads();
    uint16_t* h16 = (uint16_t*)p.h + (int64_t)r * p.ldh;
    float* h32 = (float*)p.h + (int64_t)r * p.ldh;
    fix_t* hfx = (fix_t*)p.h + (int64_t)r * p.ldh;
    float ss = 0.f;
    bool bad = false;
    for (int col = tid; col < H; col += blockDim.x) {
        float ys[8], yr[8];
#pragma unroll
        for (int s = 0; s < 8; ++s) ys[s] = s < S ? p.y[(int64_t)slot_s[8 + s] * H + col] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) yr[j] = j < K ? p.y[(int64_t)slot_s[j] * H + col] : 0.f;
        float acc = 0.f;
#pragma unroll
        for (int s = 0; s < 8; ++s) acc += ys[s];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc = fmaf(j < K ? w_s[j] : 0.f, yr[j], acc);
        float hr;
        if (p.h_mode == RESID_FIX) {
            const fix_t hv = (p.add_residual ? hfx[col] : 0) + fix_from(acc, bad);
            hfx[col] = hv;
            hr = fix_to(hv);
        } else if (p.h_mode == RESID_F32) {
            hr = p.add_residual ? h32[col] + acc : acc;
            h32[col] = hr;
        } else {
            const uint16_t hb = f2h(p.add_residual ? h2f(h16[col]) + acc : acc);
            h16[col] = hb;
            hr = h2f(hb);
        }
        ss = fmaf(hr, hr, ss);
    }
    report_status(p.status, bad, kStatResidual);
    if (!p.norm_w) return;
    ss = wave_sum(ss);
    if ((tid & 63) == 0) red[tid >> 6] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) tot += red[i];
    const float inv = 1.0f / sqrtf(tot / (float)H + p.eps);
    uint16_t* x = p.x_out + (int64_t)r * p.ldx;
    for (int col = tid; col < H; col += blockDim.x) {
        const float hv = p.h_mode == RESID_FIX ? fix_to(hfx[col]) : p.h_mode == RESID_F32 ? h32[col] : h2f(h16[col]);
        x[col] = f2h(hv * inv * h2f(p.norm_w[col]));
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Entries of the work list: decode-sized batches split every expert's tokens
// into blocks of 16 (shared experts: ceil(rows/16) blocks); larger batches
// keep one entry per active expert.
bool moe_small(int rows, const ocrdec_moe_weights* w) {
    const int E = w->n_experts, K = w->top_k, H = w->hidden;
    return rows <= 32 && E % 16 == 0 && E <= 256 && rows * K <= 256 && route_lds_bytes(rows, H) <= 96 * 1024;
}
static bool eg_format(int fmt) { return fmt == OCRDEC_F16 || fmt == OCRDEC_Q8_0 || fmt == OCRDEC_Q4_0; }
// Large batches go through the expert GEMM when every matrix format has it.
bool moe_gemm_path(int rows, const ocrdec_moe_weights* w) {
    return !moe_small(rows, w) && w->n_experts % 16 == 0 && w->hidden % EG_KS == 0 && w->d_ff % EG_KS == 0 &&
           eg_format(w->router.fmt) && eg_format(w->gate_up.fmt) && eg_format(w->down.fmt) && (w->n_shared == 0 || (eg_format(w->sh_gate_up.fmt) && eg_format(w->sh_down.fmt)));
}
// Router GEMM k-slices for large batches: about two 128-column stages per
// slice, at most eight slices, none of them empty (the kernel gives slice z
// the stages [z * ceil(n / slices), ...)).
int router_kslices(int hidden) {
    const int n = std::max(1, hidden / EG_KS), k0 = std::max(2, (n + 7) / 8);
    return (n + k0 - 1) / k0;
}

int moe_max_virt(int rows, const ocrdec_moe_weights* w) {
    const int E = w->n_experts, S = w->n_shared, NP = rows * w->top_k;
    if (moe_small(rows, w)) return S * ((rows + 15) / 16) + std::min(E, NP) + NP / 16;
    if (moe_gemm_path(rows, w)) return S * ((rows + EG_TM - 1) / EG_TM) + std::min(E, NP) + NP / EG_TM;
    return std::min(E, NP) + S;
}

MoeWs carve_moe(void* ws, int rows, const ocrdec_moe_weights* w) {
    Carve cv(ws);
    MoeWs m;
    const int NP = rows * w->top_k, E = w->n_experts, S = w->n_shared;
    const int nslots = NP + S * rows;
    m.logits = cv.take<float>((size_t)rows * E * (moe_gemm_path(rows, w) ? router_kslices(w->hidden) : 1));
    m.idx = cv.take<int32_t>(NP);
    m.w = cv.take<float>(NP);
    m.rank = cv.take<int32_t>(NP);
    m.hist = cv.take<int32_t>((size_t)((NP + 63) / 64) * E);
    m.counts = cv.take<int32_t>(E);
    m.offsets = cv.take<int32_t>(E + 1);
    m.perm = cv.take<int32_t>(NP);
    m.inv = cv.take<int32_t>(NP);
    m.vrows = cv.take<int32_t>(nslots);
    m.n_virt = cv.take<int32_t>(1);
    m.virt = cv.take<int4>(moe_max_virt(rows, w));
    m.a = cv.take<uint16_t>((size_t)nslots * w->d_ff);
    m.y = cv.take<float>((size_t)nslots * w->hidden);
    m.sw = cv.take<float>(nslots);
    m.bytes = cv.off;
    return m;
}

ocrdec_status check_moe(const ocrdec_moe_weights* w, int rows) {
    OCR_CHECK_ARG(w, "weights is NULL");
    OCR_CHECK_ARG(rows >= 1 && rows <= 65536, "rows must be in [1, 65536]");
    OCR_CHECK_ARG(w->hidden > 0 && w->hidden % 32 == 0 && w->hidden <= 4096,
                  "hidden must be a positive multiple of 32, at most 4096");
    OCR_CHECK_ARG(w->d_ff > 0 && w->d_ff % 32 == 0, "d_ff must be a positive multiple of 32");
    if (w->n_experts < 1 || w->n_experts > 256) return fail(OCRDEC_ERR_UNSUPPORTED, "n_experts must be in [1, 256]");
    if (w->top_k < 1 || w->top_k > 8 || w->top_k > w->n_experts)
        return fail(OCRDEC_ERR_UNSUPPORTED, "top_k must be in [1, min(8, n_experts)]");
    OCR_CHECK_ARG(w->n_shared >= 0 && w->n_shared <= 8, "n_shared must be in [0, 8]");
    ocrdec_status s;
    if ((s = check_qmat(&w->router, "router")) != OCRDEC_OK) return s;
    if ((s = check_qmat(&w->gate_up, "gate_up")) != OCRDEC_OK) return s;
    if ((s = check_qmat(&w->down, "down")) != OCRDEC_OK) return s;
    OCR_CHECK_ARG(w->router.n == w->n_experts && w->router.k == w->hidden, "router must be [n_experts][hidden]");
    OCR_CHECK_ARG(w->gate_up.n == w->n_experts * 2 * w->d_ff && w->gate_up.k == w->hidden,
                  "gate_up must be [n_experts*2*d_ff][hidden]");
    OCR_CHECK_ARG(w->down.n == w->n_experts * w->hidden && w->down.k == w->d_ff, "down must be [n_experts*hidden][d_ff]");
    if (w->n_shared > 0) {
        if ((s = check_qmat(&w->sh_gate_up, "sh_gate_up")) != OCRDEC_OK) return s;
        if ((s = check_qmat(&w->sh_down, "sh_down")) != OCRDEC_OK) return s;
        OCR_CHECK_ARG(w->sh_gate_up.n == w->n_shared * 2 * w->d_ff && w->sh_gate_up.k == w->hidden,
                      "sh_gate_up must be [n_shared*2*d_ff][hidden]");
        OCR_CHECK_ARG(w->sh_down.n == w->n_shared * w->hidden && w->sh_down.k == w->d_ff,
                      "sh_down must be [n_shared*hidden][d_ff]");
        if (w->sh_gate_up.fmt != w->gate_up.fmt || w->sh_down.fmt != w->down.fmt)
            return fail(OCRDEC_ERR_UNSUPPORTED, "shared and routed experts must use the same formats");
    }
    return OCRDEC_OK;
}

namespace {

template <int FMT, bool GLU>
void launch_grouped_fmt(const GroupedParams& p, int xt, int ks, bool lds, int grid, hipStream_t s) {
    const size_t lb = lds ? lds_x_bytes(p.k, xt) : 0;
    if (p.pidx) {
        // expert-indexed entries (16 tokens, one wave per item); the down
        // projection adds into the residual
        if (lds) hipLaunchKernelGGL((grouped_kernel<FMT, 1, 1, GLU, true, !GLU, true>), dim3(grid), dim3(256), lb, s, p);
        else hipLaunchKernelGGL((grouped_kernel<FMT, 1, 1, GLU, false, !GLU, true>), dim3(grid), dim3(256), 0, s, p);
        return;
    }
#define OCR_G(XT_, KS_)                                                                                          \
    if (xt == XT_ && ks == KS_) {                                                                               \
        if (!GLU && p.sw) {                                                                                     \
            if (lds) hipLaunchKernelGGL((grouped_kernel<FMT, XT_, KS_, GLU, true, !GLU>), dim3(grid), dim3(256), lb, s, p); \
            else hipLaunchKernelGGL((grouped_kernel<FMT, XT_, KS_, GLU, false, !GLU>), dim3(grid), dim3(256), 0, s, p);    \
        } else if (lds) {                                                                                       \
            hipLaunchKernelGGL((grouped_kernel<FMT, XT_, KS_, GLU, true>), dim3(grid), dim3(256), lb, s, p);     \
        } else {                                                                                                \
            hipLaunchKernelGGL((grouped_kernel<FMT, XT_, KS_, GLU, false>), dim3(grid), dim3(256), 0, s, p);     \
        }                                                                                                       \
        return;                                                                                                 \
    }
    OCR_G(1, 1) OCR_G(2, 1) OCR_G(1, 4) OCR_G(2, 4)
#undef OCR_G
}

// Streamed form (grouped_stream_kernel): two items per wave, entries of at
// most 16 tokens staged in LDS; the ring depth must divide the stream.
constexpr int STREAM_IPW = 2;
inline int stream_pf(bool glu) { return glu ? 5 : 7; }
// LDS of the streamed kernels: 16 staged rows, then (Q4_0) 16 floats per
// 32-column block
inline size_t stream_lds_bytes(int k) { return lds_x_bytes(k, 1) + (size_t)(k / 32) * 64; }
inline bool stream_ok(const GroupedParams& p, bool glu) {
    return p.groups_per_expert % (4 * STREAM_IPW) == 0 && stream_lds_bytes(p.k) <= 65536 && p.k % 128 == 0 &&
           (STREAM_IPW * p.nchunks) % stream_pf(glu) == 0;
}
template <int FMT, bool GLU>
void launch_stream_t(const GroupedParams& p, hipStream_t s) {
    constexpr int PF = GLU ? 5 : 7;  // = stream_pf(GLU)
    const int grid = p.max_virt * (p.groups_per_expert / (4 * STREAM_IPW));
    const size_t lb = stream_lds_bytes(p.k);
    if (p.pidx) {
        if (GLU) hipLaunchKernelGGL((grouped_stream_kernel<FMT, GLU, false, STREAM_IPW, PF, true>), dim3(grid), dim3(256), lb, s, p);
        else hipLaunchKernelGGL((grouped_stream_kernel<FMT, GLU, true, STREAM_IPW, PF, true>), dim3(grid), dim3(256), lb, s, p);
    } else if (!GLU && p.sw) hipLaunchKernelGGL((grouped_stream_kernel<FMT, GLU, true, STREAM_IPW, PF>), dim3(grid), dim3(256), lb, s, p);
    else hipLaunchKernelGGL((grouped_stream_kernel<FMT, GLU, false, STREAM_IPW, PF>), dim3(grid), dim3(256), lb, s, p);
}

void launch_grouped(int fmt, bool glu, GroupedParams p, int rows_hint, hipStream_t s) {
    const int64_t items = (int64_t)p.max_virt * p.groups_per_expert;
    // (expert-indexed entries: one wave per item)
    const int ks = (items >= 2048 || p.pidx) ? 1 : 4;
    // gate/up of decode batches from 6 rows: the streamed form (entries of at
    // most 16 tokens, staged in LDS).  It halves the workgroups, which pays
    // once they exceed the CUs' workgroup slots (two per CU for the one-item
    // form), and its Q4_0 loop (biased codes) has the fewest VALU operations
    // per weight: gate/up 15.3 -> 13.5 us at 6 rows, 17.4 -> 15.7 at 8.
    if (glu && rows_hint >= 6 && p.entries16 && ks == 1 && stream_ok(p, true) && use_lds_x(p.k, 1, rows_hint)) {
        switch (fmt) {
        case OCRDEC_F16: launch_stream_t<OCRDEC_F16, true>(p, s); return;
        case OCRDEC_Q8_0: launch_stream_t<OCRDEC_Q8_0, true>(p, s); return;
        case OCRDEC_Q4_0: launch_stream_t<OCRDEC_Q4_0, true>(p, s); return;
        case OCRDEC_U8A_G32: launch_stream_t<OCRDEC_U8A_G32, true>(p, s); return;
        }
    }
    // the expert-indexed down projection of 20 or more rows: the streamed form
    // too (24 rows: 20.0 -> 19.0 us; slower at 6 and 12 rows, 12.1 -> 14.6 and
    // 14.1 -> 15.3 us)
    if (!glu && p.pidx && rows_hint >= 20 && stream_ok(p, false)) {
        switch (fmt) {
        case OCRDEC_F16: launch_stream_t<OCRDEC_F16, false>(p, s); return;
        case OCRDEC_Q8_0: launch_stream_t<OCRDEC_Q8_0, false>(p, s); return;
        case OCRDEC_Q4_0: launch_stream_t<OCRDEC_Q4_0, false>(p, s); return;
        case OCRDEC_U8A_G32: launch_stream_t<OCRDEC_U8A_G32, false>(p, s); return;
        }
    }
    // LDS staging needs every wave of a workgroup on the same expert; it uses
    // 16-token passes (routed experts usually get far fewer tokens than rows)
    const bool same_expert = (p.groups_per_expert % (4 / ks)) == 0;
    // the down projection reads its activations contiguously: LDS staging pays
    // for any row count there (and keeps three workgroups per CU)
    const bool lds = (glu ? use_lds_x(p.k, 1, rows_hint) : lds_x_bytes(p.k, 1) <= 65536) && same_expert;
    const int xt = (lds || p.pidx) ? 1 : (rows_hint <= 16 ? 1 : 2);
    const int grid = (int)((items + (4 / ks) - 1) / (4 / ks));
#define OCR_F(F_)                                                                          \
    case F_:                                                                               \
        if (glu) launch_grouped_fmt<F_, true>(p, xt, ks, lds, grid, s);                    \
        else launch_grouped_fmt<F_, false>(p, xt, ks, lds, grid, s);                       \
        break;
    switch (fmt) {
        OCR_F(OCRDEC_F16)
        OCR_F(OCRDEC_Q8_0)
        OCR_F(OCRDEC_Q4_0)
        OCR_F(OCRDEC_U8A_G32)
    }
#undef OCR_F
}

template <int FMT, bool GLU>
void launch_eg_t(const GroupedParams& p, int n_entries, hipStream_t s) {
    const int cgs = GLU ? (p.out_tiles + EG_NW - 1) / EG_NW : (p.out_tiles + 2 * EG_NW - 1) / (2 * EG_NW);
    // every XCD gets room for cgs * ceil(n_entries / 8) work items
    const int grid = 8 * cgs * std::max(p.kslices, 1) * ((n_entries + 7) / 8);
    hipLaunchKernelGGL((expert_gemm_kernel<FMT, GLU>), dim3(grid), dim3(64 * EG_NW), EG_LDS, s, p, cgs);
}

void launch_expert_gemm(int fmt, bool glu, const GroupedParams& p, int n_entries, hipStream_t s) {
#define OCR_EG(F_)                                               \
    case F_:                                                     \
        if (glu) launch_eg_t<F_, true>(p, n_entries, s);         \
        else launch_eg_t<F_, false>(p, n_entries, s);            \
        break;
    switch (fmt) {
        OCR_EG(OCRDEC_F16)
        OCR_EG(OCRDEC_Q8_0)
        OCR_EG(OCRDEC_Q4_0)
    }
#undef OCR_EG
}

}  // namespace

bool dense_gemm_ok(int fmt, int n, int k, int rows, int64_t ldx) {
    return eg_format(fmt) && k % EG_KS == 0 && n % 16 == 0 && rows >= 1 && (int64_t)(rows - 1) * ldx + k < (1ll << 30);
}

void launch_dense_gemm(int fmt, bool glu, const uint8_t* w, int n, int k, int rows, const uint16_t* x, int64_t ldx,
                       void* y, int64_t ldy, hipStream_t s) {
    GroupedParams p{};
    p.w_routed = w;
    p.n_experts = 1;
    p.k = k;
    p.nchunks = n_chunks(fmt, k);
    p.out_tiles = n / 16;
    p.dense_rows = rows;
    p.x = x;
    p.ldx = ldx;
    p.y = y;
    p.ldy = ldy;
    launch_expert_gemm(fmt, glu, p, (rows + EG_TM - 1) / EG_TM, s);
}

// Work entries of the expert-indexed decode MoE: (shared experts, then
// routed ones) x 16-token blocks, tokens found from the chosen experts.
static void set_byexp(GroupedParams& p, const MoeWs& m, int rows, int K, int S) {
    p.pidx = m.idx;
    p.pw = m.w;
    p.rows = rows;
    p.top_k = K;
    p.nb16 = (rows + 15) / 16;
    p.n_shared = S;
    p.max_virt = (p.n_experts + S) * p.nb16;
}

void launch_moe(const ocrdec_moe_weights* w, int rows, const uint16_t* x, int64_t ldx, void* h, int h_mode, int64_t ldh,
                int add_residual, const int32_t* forced, const ocrdec_moe_capture* cap, int32_t* cap_idx,
                float* cap_w, const MoeWs& m, const uint16_t* norm_w, float eps, uint16_t* x_out, int64_t ldxo,
                hipStream_t s, const fix_t* h_norm, const uint16_t* norm_in, float eps_in, bool fuse_combine,
                uint32_t* status) {
    const int E = w->n_experts, K = w->top_k, S = w->n_shared, F = w->d_ff, H = w->hidden;
    const int NP = rows * K;
    MoeParams p{};
    p.rows = rows;
    p.n_experts = E;
    p.top_k = K;
    p.n_shared = S;
    p.logits = m.logits;
    p.bias = w->router_bias;
    p.forced = forced;
    p.idx = m.idx;
    p.w = m.w;
    p.rank = m.rank;
    p.hist = m.hist;
    p.counts = m.counts;
    p.offsets = m.offsets;
    p.perm = m.perm;
    p.inv = m.inv;
    p.vrows = m.vrows;
    p.n_virt = m.n_virt;
    p.virt = m.virt;
    p.cap_idx = cap_idx ? cap_idx : (cap ? cap->topk_idx : nullptr);
    p.cap_w = cap_w ? cap_w : (cap ? cap->topk_w : nullptr);
    p.cap_counts = cap ? cap->counts : nullptr;
    p.cap_offsets = cap ? cap->offsets : nullptr;
    p.cap_perm = cap ? cap->perm : nullptr;
    const bool small = moe_small(rows, w);
    // the expert GEMM addresses its activations with 32-bit byte offsets
    const bool gemm = moe_gemm_path(rows, w) && (int64_t)(rows - 1) * ldx + H < (1ll << 30) &&
                      (int64_t)(NP + S * rows) * F < (1ll << 30);
    // decode-sized batches with the fixed-point residual: the down projection
    // adds its weighted outputs into the residual itself (atomic integer adds),
    // no combine kernel
    const bool fused = fuse_combine && small && h_mode == RESID_FIX && add_residual;
    // 2-32 rows of the decode step: the expert-indexed form.  One routing
    // workgroup per row (norm, router GEMV, top-k), no grouping pass; each
    // expert kernel workgroup owns a fixed (expert, 16-token block) and finds
    // its tokens in the chosen experts itself.  (One row keeps the single
    // routing workgroup, whose grouping of one row is a few lane operations.)
    const bool byexp = fused && rows >= 2 && !p.cap_counts && !p.cap_offsets && !p.cap_perm &&
                       (F / 16) % (4 * 2) == 0 && (H / 16) % 4 == 0;
    // the grouping also lists every slot's combine weight: the down projection
    // adds its outputs into the residual itself
    if (fused && !byexp) p.sw = m.sw;
    if (norm_in && !small) {
        // the MoE input is the normalised residual: form it first
        prof_mark(s, OCRDEC_K_NORM);
        hipLaunchKernelGGL(moe_norm_kernel, dim3(rows), dim3(256), 0, s, h_norm, norm_in, H, eps_in, (uint16_t*)x,
                           ldx);
    }
    prof_mark(s, OCRDEC_K_ROUTE);
    if (small) {
        // router GEMV, top-k and grouping in one workgroup
        const uint8_t* rw = (const uint8_t*)w->router.data;
        // 17-32 rows: one 32-token pass over the router weights where the LDS
        // allows (fp16 and Q8_0 routers; the other formats' variants spill)
        const bool xt2 = !byexp && rows > 16 && route_lds_bytes(rows, H) <= 84 * 1024 &&
                         (w->router.fmt == OCRDEC_F16 || w->router.fmt == OCRDEC_Q8_0);
#define OCR_RLB(F_, NV_, B_)                                                                                   \
    if (byexp)                                                                                                 \
        hipLaunchKernelGGL((route_fused_kernel<F_, NV_, B_, 1, ROUTE_ROW>), dim3(rows), dim3(1024), route_lds_bytes(1, H), \
                           s, p, rw, H, x, ldx, h_norm, norm_in, eps_in, (uint16_t*)x);                        \
    else if (rows == 1)                                                                                        \
        hipLaunchKernelGGL((route_fused_kernel<F_, NV_, B_, 1, ROUTE_ONE>), dim3(1), dim3(1024), route_lds_bytes(1, H), \
                           s, p, rw, H, x, ldx, h_norm, norm_in, eps_in, (uint16_t*)x);                        \
    else if (xt2)                                                                                              \
        hipLaunchKernelGGL((route_fused_kernel<F_, NV_, B_, 2>), dim3(1), dim3(1024), route_lds_bytes(rows, H), s, p, \
                           rw, H, x, ldx, h_norm, norm_in, eps_in, (uint16_t*)x);                              \
    else                                                                                                       \
        hipLaunchKernelGGL((route_fused_kernel<F_, NV_, B_, 1>), dim3(1), dim3(1024), route_lds_bytes(rows, H), s, p, \
                           rw, H, x, ldx, h_norm, norm_in, eps_in, (uint16_t*)x)
#define OCR_RL(F_, NV_)                 \
    do {                                \
        if (p.bias) {                   \
            OCR_RLB(F_, NV_, true);     \
        } else {                        \
            OCR_RLB(F_, NV_, false);    \
        }                               \
    } while (0)
#define OCR_R(F_)                      \
    case F_:                           \
        if (H <= 1280) OCR_RL(F_, 5);  \
        else if (H <= 2048) OCR_RL(F_, 8); \
        else OCR_RL(F_, 16);           \
        break;
        switch (w->router.fmt) {
            OCR_R(OCRDEC_F16)
            OCR_R(OCRDEC_Q8_0)
            OCR_R(OCRDEC_Q4_0)
            OCR_R(OCRDEC_U8A_G32)
        }
#undef OCR_R
#undef OCR_RL
#undef OCR_RLB
    } else if (gemm) {
        // router GEMM, parallel top-k, grouping into 128-token entries
        GroupedParams rp{};
        rp.w_routed = (const uint8_t*)w->router.data;
        rp.n_experts = 1;
        rp.k = H;
        rp.nchunks = n_chunks(w->router.fmt, H);
        rp.out_tiles = E / 16;
        rp.dense_rows = rows;
        rp.x = x;
        rp.ldx = ldx;
        rp.y = m.logits;
        rp.ldy = E;
        rp.kslices = router_kslices(H);  // few entries: the k range is split over workgroups
        rp.ly_slice = (int64_t)rows * E;
        p.lslices = rp.kslices;
        p.lslice = rp.ly_slice;
        launch_expert_gemm(w->router.fmt, false, rp, (rows + EG_TM - 1) / EG_TM, s);
        prof_mark(s, OCRDEC_K_ROUTE);
        hipLaunchKernelGGL(topk_kernel, dim3((rows + 15) / 16), dim3(1024), 0, s, p);
        prof_mark(s, OCRDEC_K_ROUTE);
        hipLaunchKernelGGL(group_large_kernel, dim3(1), dim3(1024), 0, s, p, EG_TM);
    } else {
        GemvPlan pl = plan_gemv(w->router.fmt, E, H, rows, EPI_F32);
        GemvParams gp{};
        gp.w = (const uint8_t*)w->router.data;
        gp.n = E;
        gp.k = H;
        gp.nchunks = n_chunks(w->router.fmt, H);
        gp.xs = XDirect{x, ldx, rows};
        gp.y = m.logits;
        gp.ldy = E;
        launch_gemv(w->router.fmt, EPI_F32, pl, gp, s);
        prof_mark(s, OCRDEC_K_ROUTE);
        hipLaunchKernelGGL(route_group_kernel, dim3(1), dim3(1024), 0, s, p);
    }
    const int max_virt = moe_max_virt(rows, w);
    // gate/up with SwiGLU
    {
        GroupedParams p{};
        p.w_routed = (const uint8_t*)w->gate_up.data;
        p.w_shared = S ? (const uint8_t*)w->sh_gate_up.data : nullptr;
        p.n_experts = E;
        p.k = H;
        p.nchunks = n_chunks(w->gate_up.fmt, H);
        p.expert_bytes = (int64_t)(2 * F / 16) * p.nchunks * pack_cb(w->gate_up.fmt);
        p.half_tiles = F / 16;
        p.groups_per_expert = F / 16;
        p.max_virt = max_virt;
        p.n_virt = m.n_virt;
        p.virt = m.virt;
        p.vrows = m.vrows;
        p.np = NP;
        p.x = x;
        p.ldx = ldx;
        p.y = m.a;
        p.ldy = F;
        p.out_tiles = F / 16;
        p.one_row = rows == 1;
        p.entries16 = small;
        if (byexp) set_byexp(p, m, rows, K, S);
        prof_mark(s, OCRDEC_K_EXPERT_GLU);
        if (gemm) launch_expert_gemm(w->gate_up.fmt, true, p, max_virt, s);
        else launch_grouped(w->gate_up.fmt, true, p, rows, s);
    }
    // down
    {
        GroupedParams p{};
        p.w_routed = (const uint8_t*)w->down.data;
        p.w_shared = S ? (const uint8_t*)w->sh_down.data : nullptr;
        p.n_experts = E;
        p.k = F;
        p.nchunks = n_chunks(w->down.fmt, F);
        p.expert_bytes = (int64_t)(H / 16) * p.nchunks * pack_cb(w->down.fmt);
        p.half_tiles = 0;
        p.groups_per_expert = H / 16;
        p.max_virt = max_virt;
        p.n_virt = m.n_virt;
        p.virt = m.virt;
        p.vrows = m.vrows;
        p.np = NP;
        p.x = m.a;
        p.ldx = F;
        p.y = m.y;
        p.ldy = H;
        p.out_tiles = H / 16;
        p.one_row = rows == 1;
        p.entries16 = small;
        if (fused) {
            p.sw = m.sw;
            p.h = (fix_t*)h;
            p.ldh = ldh;
            p.status = status;
        }
        if (byexp) set_byexp(p, m, rows, K, S);
        prof_mark(s, OCRDEC_K_EXPERT_DOWN);
        if (gemm) launch_expert_gemm(w->down.fmt, false, p, max_virt, s);
        else launch_grouped(w->down.fmt, false, p, rows, s);
    }
    // combine, or (down projection added into the residual) the next norm
    if (fused) {
        if (norm_w) prof_mark(s, OCRDEC_K_NORM);
        if (norm_w)
            hipLaunchKernelGGL(moe_norm_kernel, dim3(rows), dim3(256), 0, s, (const fix_t*)h, norm_w, H, eps, x_out,
                               ldxo);
    } else {
        CombineParams p{};
        p.rows = rows;
        p.hidden = H;
        p.top_k = K;
        p.n_shared = S;
        p.np = NP;
        p.w = m.w;
        p.inv = m.inv;
        p.y = m.y;
        p.h = h;
        p.h_mode = h_mode;
        p.status = status;
        p.ldh = ldh;
        p.add_residual = add_residual;
        p.norm_w = norm_w;
        p.eps = eps;
        p.x_out = x_out;
        p.ldx = ldxo;
        prof_mark(s, OCRDEC_K_COMBINE);
        hipLaunchKernelGGL(combine_kernel, dim3(rows), dim3(rows <= 64 ? 1024 : 256), 0, s, p);
    }
}

}  // namespace ocrdec

using namespace ocrdec;

extern "C" ocrdec_status ocrdec_moe_workspace_bytes(const ocrdec_moe_weights* w, int32_t rows, size_t* bytes) {
    ocrdec_status st = check_moe(w, rows);
    if (st != OCRDEC_OK) return st;
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    *bytes = carve_moe(nullptr, rows, w).bytes;
    return OCRDEC_OK;
}

extern "C" ocrdec_status ocrdec_moe_layer(const ocrdec_moe_weights* w, int32_t rows, const uint16_t* x, uint16_t* h,
                                          int32_t add_residual, const int32_t* forced_topk,
                                          const ocrdec_moe_capture* capture, void* ws, size_t ws_bytes,
                                          void* stream) {
    ocrdec_status st = check_moe(w, rows);
    if (st != OCRDEC_OK) return st;
    OCR_CHECK_ARG(x && h, "x and h must be non-NULL");
    OCR_CHECK_ARG(((uintptr_t)x & 15) == 0, "x must be 16-byte aligned");
    const size_t need = carve_moe(nullptr, rows, w).bytes;
    if (!ws || ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "MoE workspace: need " + std::to_string(need) + " bytes, got " +
                                              std::to_string(ws ? ws_bytes : 0));
    MoeWs m = carve_moe(ws, rows, w);
    launch_moe(w, rows, x, w->hidden, h, RESID_F16, w->hidden, add_residual, forced_topk, capture, nullptr, nullptr, m, nullptr,
               0.f, nullptr, 0, (hipStream_t)stream, nullptr, nullptr, 0.f);
    return launch_status("ocrdec_moe_layer");
}

// A decode round: a queue of requests served by the rows of one decode
// state ("Nicolassuez/Falcon-OCR-int8-openvino", "How it is meant to be run":
// a decode step reads all the weights to advance one token, so rows share
// that read, and merging several requests into one round is what makes a
// queue affordable; "HunyuanOCR 的 ncnn 移植" 3.5: generation stops at any
// token of the EOS set, before the token is handed out).
//
// Each request gets a free row (lowest first, requests in order); the prompt
// passes of the requests admitted together run as one batch (their inputs
// packed into the workspace), fill the rows' cache prefixes and give the
// first tokens; then one decode step over the occupied rows advances all of
// them together.  After every step the host reads the new tokens and retires
// the rows that reached an EOS token or their token budget; freed rows take
// the next requests.
#include <algorithm>
#include <vector>

#include "common.hpp"

namespace ocrdec {
namespace {

struct Admitted {
    int n;
    int row[32];
    int P[32];
};

// rows admitted together: prefix_len = P, generation index 0, and the first
// token of sequence i (tok_first[i]) into the row's token slot
__global__ void admit_rows_kernel(int32_t* prefix_len, int32_t* gen_index, int32_t* tok, const int32_t* tok_first,
                                  Admitted a) {
    const int i = threadIdx.x;
    if (i < a.n) {
        prefix_len[a.row[i]] = a.P[i];
        gen_index[a.row[i]] = 0;
        tok[a.row[i]] = tok_first[i];
    }
}

// workspace: the row tokens, the first tokens of a batch, the packed prompt
// tokens and features of up to `rows` requests, then the larger of the
// batched prompt-pass and step workspaces
struct RoundWs {
    int32_t* tok;
    int32_t* first;
    int32_t* ptok;
    uint16_t* pemb;
    char* inner;
    size_t inner_bytes;
    size_t bytes;
};

RoundWs carve_round(void* ws, int rows, int max_P, int H, size_t inner_bytes) {
    Carve cv(ws);
    RoundWs w;
    w.tok = cv.take<int32_t>(rows);
    w.first = cv.take<int32_t>(rows);
    w.ptok = cv.take<int32_t>((size_t)rows * max_P);
    w.pemb = cv.take<uint16_t>((size_t)rows * max_P * H);
    w.inner = cv.take<char>(inner_bytes);
    w.inner_bytes = inner_bytes;
    w.bytes = cv.off;
    return w;
}

}  // namespace
}  // namespace ocrdec

using namespace ocrdec;

namespace {
ocrdec_status round_sizes(const ocrdec_model* m, const ocrdec_state* st, int max_P, size_t* inner, size_t* total) {
    OCR_CHECK_ARG(m && st, "model and state must be non-NULL");
    OCR_CHECK_ARG(st->rows >= 1 && st->rows <= 32, "rows must be in [1, 32]");
    std::vector<int32_t> rows(st->rows), P(st->rows, max_P);
    for (int i = 0; i < st->rows; ++i) rows[i] = i;
    size_t pre = 0, step = 0;
    ocrdec_status s;
    if ((s = ocrdec_prefill_batch_workspace_bytes(m, st, st->rows, rows.data(), P.data(), &pre)) != OCRDEC_OK) return s;
    if ((s = ocrdec_step_workspace_bytes(m, st, &step)) != OCRDEC_OK) return s;
    *inner = std::max(pre, step);
    *total = carve_round(nullptr, st->rows, max_P, m->hidden, *inner).bytes;
    return OCRDEC_OK;
}
}  // namespace

extern "C" ocrdec_status ocrdec_round_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st, int32_t max_P,
                                                      size_t* bytes) {
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    size_t inner = 0;
    return round_sizes(m, st, max_P, &inner, bytes);
}

extern "C" ocrdec_status ocrdec_run_round(const ocrdec_model* m, const ocrdec_state* st, ocrdec_request* reqs,
                                          int32_t n_reqs, const int32_t* eos, int32_t n_eos, int32_t keep_eos,
                                          void* ws, size_t ws_bytes, void* stream) {
    OCR_CHECK_ARG(m && st, "model and state must be non-NULL");
    OCR_CHECK_ARG(n_reqs >= 0 && (reqs || n_reqs == 0), "reqs is NULL");
    OCR_CHECK_ARG(n_eos >= 0 && (eos || n_eos == 0), "eos is NULL");
    OCR_CHECK_ARG(m->lm_head.data, "a round needs an LM head");
    int max_P = 1;
    for (int i = 0; i < n_reqs; ++i) {
        const ocrdec_request& r = reqs[i];
        const std::string tag = "request " + std::to_string(i) + ": ";
        OCR_CHECK_ARG(r.P >= 1 && r.P <= st->prefix_cap, tag + "P must be in [1, prefix_cap]");
        OCR_CHECK_ARG(r.tokens || r.features, tag + "tokens or features must be given");
        OCR_CHECK_ARG(r.max_new >= 1, tag + "max_new must be >= 1");
        OCR_CHECK_ARG(r.out, tag + "out is NULL");
        max_P = std::max(max_P, (int)r.P);
    }
    size_t need = 0, inner_need = 0;
    ocrdec_status s = round_sizes(m, st, max_P, &inner_need, &need);
    if (s != OCRDEC_OK) return s;
    if (!ws || ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "round workspace: need " + std::to_string(need) + " bytes, got " +
                                              std::to_string(ws ? ws_bytes : 0));
    hipStream_t hs = (hipStream_t)stream;
    const int rows = st->rows, H = m->hidden;
    const RoundWs W = carve_round(ws, rows, max_P, H, inner_need);
    int32_t* tok = W.tok;
    char* inner = W.inner;
    const size_t inner_bytes = W.inner_bytes;
    const std::vector<int32_t> eos_set(eos, eos + n_eos);
    auto is_eos = [&](int32_t t) { return std::find(eos_set.begin(), eos_set.end(), t) != eos_set.end(); };
    for (int i = 0; i < n_reqs; ++i) {
        reqs[i].n_out = 0;
        reqs[i].stop = 0;
    }
    std::vector<int> owner(rows, -1);  // request in each row
    std::vector<int32_t> host_tok(rows);
    int next = 0;
    // a token for request q: recorded, then the request stops at EOS or its budget
    auto take = [&](int q, int32_t t) {
        ocrdec_request& r = reqs[q];
        if (is_eos(t)) {
            if (keep_eos) r.out[r.n_out++] = t;
            r.stop = 1;
            return true;
        }
        r.out[r.n_out++] = t;
        if (r.n_out >= r.max_new) {
            r.stop = 2;
            return true;
        }
        return false;
    };
    auto read_tokens = [&](int n) -> ocrdec_status {
        if (hipMemcpyAsync(host_tok.data(), tok, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, hs) != hipSuccess ||
            hipStreamSynchronize(hs) != hipSuccess)
            return fail(OCRDEC_ERR_DEVICE, "ocrdec_run_round: reading the tokens failed");
        return OCRDEC_OK;
    };
    for (;;) {
        // admit requests into free rows until every row is busy or the queue is empty
        bool admitted = true;
        while (admitted) {
            admitted = false;
            std::vector<int> fresh;
            for (int row = 0; row < rows && next < n_reqs; ++row) {
                if (owner[row] >= 0) continue;
                owner[row] = next++;
                fresh.push_back(row);
            }
            if (fresh.empty()) break;
            // one batched prompt pass for the token requests, one for the
            // feature requests, their inputs packed into the workspace
            for (int kind = 0; kind < 2; ++kind) {
                Admitted a{};
                std::vector<int32_t> brow, bP;
                int64_t off = 0;
                for (int row : fresh) {
                    const ocrdec_request& r = reqs[owner[row]];
                    if ((r.tokens != nullptr) != (kind == 0)) continue;
                    hipError_t e = kind == 0 ? hipMemcpyAsync(W.ptok + off, r.tokens, (size_t)r.P * sizeof(int32_t),
                                                              hipMemcpyDeviceToDevice, hs)
                                             : hipMemcpyAsync(W.pemb + off * H, r.features, (size_t)r.P * H * 2,
                                                              hipMemcpyDeviceToDevice, hs);
                    if (e != hipSuccess) return fail(OCRDEC_ERR_DEVICE, "ocrdec_run_round: packing a prompt failed");
                    off += r.P;
                    a.row[a.n] = row;
                    a.P[a.n] = r.P;
                    ++a.n;
                    brow.push_back(row);
                    bP.push_back(r.P);
                }
                if (a.n == 0) continue;
                s = ocrdec_prefill_batch(m, st, a.n, brow.data(), bP.data(), kind == 0 ? W.ptok : nullptr,
                                         kind == 0 ? nullptr : W.pemb, nullptr, W.first, nullptr, nullptr, inner,
                                         inner_bytes, stream);
                if (s != OCRDEC_OK) return s;
                prof_mark(hs, OCRDEC_K_OTHER);
                hipLaunchKernelGGL(admit_rows_kernel, dim3(1), dim3(64), 0, hs, (int32_t*)st->prefix_len,
                                   st->gen_index, tok, W.first, a);
            }
            if ((s = launch_status("ocrdec_run_round")) != OCRDEC_OK) return s;
            if ((s = read_tokens(rows)) != OCRDEC_OK) return s;
            for (int row : fresh)
                if (take(owner[row], host_tok[row])) {
                    owner[row] = -1;
                    admitted = true;  // the row is free again
                }
        }
        int used = 0;
        for (int row = 0; row < rows; ++row)
            if (owner[row] >= 0) used = row + 1;
        if (used == 0) break;
        // one decode step over rows [0, used): free rows in between compute
        // on whatever they hold, which nothing reads
        ocrdec_state sub = *st;
        sub.rows = used;
        s = ocrdec_decode_step(m, &sub, tok, nullptr, tok, nullptr, nullptr, inner, inner_bytes, stream);
        if (s != OCRDEC_OK) return s;
        if ((s = read_tokens(used)) != OCRDEC_OK) return s;
        for (int row = 0; row < used; ++row)
            if (owner[row] >= 0 && take(owner[row], host_tok[row])) owner[row] = -1;
    }
    return OCRDEC_OK;
}

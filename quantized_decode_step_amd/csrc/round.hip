// A decode round: a queue of requests served by the rows of one decode
// state ("Nicolassuez/Falcon-OCR-int8-openvino", "How it is meant to be run":
// a decode step reads all the weights to advance one token, so rows share
// that read, and merging several requests into one round is what makes a
// queue affordable; "HunyuanOCR 的 ncnn 移植" 3.5: generation stops at any
// token of the EOS set, before the token is handed out).
//
// Each request gets a free row (lowest first, requests in order), its prompt
// pass fills the row's cache prefix and gives the first token, then one
// decode step over the occupied rows advances all of them together.  After
// every step the host reads the new tokens and retires the rows that reached
// an EOS token or their token budget; freed rows take the next requests.
#include <algorithm>
#include <vector>

#include "common.hpp"

namespace ocrdec {
namespace {

__global__ void admit_row_kernel(int32_t* prefix_len, int32_t* gen_index, int row, int P) {
    if (threadIdx.x == 0) {
        prefix_len[row] = P;
        gen_index[row] = 0;
    }
}

}  // namespace
}  // namespace ocrdec

using namespace ocrdec;

extern "C" ocrdec_status ocrdec_round_workspace_bytes(const ocrdec_model* m, const ocrdec_state* st, int32_t max_P,
                                                      size_t* bytes) {
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    size_t pre = 0, step = 0;
    ocrdec_status s;
    if ((s = ocrdec_prefill_workspace_bytes(m, st, max_P, &pre)) != OCRDEC_OK) return s;
    if ((s = ocrdec_step_workspace_bytes(m, st, &step)) != OCRDEC_OK) return s;
    *bytes = align256((size_t)st->rows * sizeof(int32_t)) + std::max(pre, step);
    return OCRDEC_OK;
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
    size_t need = 0;
    ocrdec_status s = ocrdec_round_workspace_bytes(m, st, max_P, &need);
    if (s != OCRDEC_OK) return s;
    if (!ws || ws_bytes < need)
        return fail(OCRDEC_ERR_WORKSPACE, "round workspace: need " + std::to_string(need) + " bytes, got " +
                                              std::to_string(ws ? ws_bytes : 0));
    hipStream_t hs = (hipStream_t)stream;
    const int rows = st->rows;
    int32_t* tok = (int32_t*)ws;
    char* inner = (char*)ws + align256((size_t)rows * sizeof(int32_t));
    const size_t inner_bytes = ws_bytes - align256((size_t)rows * sizeof(int32_t));
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
                const ocrdec_request& r = reqs[next];
                ocrdec_state one = *st;
                s = ocrdec_prefill(m, &one, row, r.P, r.tokens, r.tokens ? nullptr : r.features, nullptr, tok + row,
                                   nullptr, nullptr, inner, inner_bytes, stream);
                if (s != OCRDEC_OK) return s;
                hipLaunchKernelGGL(admit_row_kernel, dim3(1), dim3(64), 0, hs, (int32_t*)st->prefix_len, st->gen_index,
                                   row, r.P);
                owner[row] = next++;
                fresh.push_back(row);
            }
            if (fresh.empty()) break;
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

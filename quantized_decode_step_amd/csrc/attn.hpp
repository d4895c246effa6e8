// Host-side interface of the decode-attention kernels.
#pragma once

#include "common.hpp"

namespace ocrdec {

struct AttnParams {
    int rows, n_heads, head_dim;
    const float* qkv;
    int64_t ld_qkv;
    uint16_t* k_cache;
    uint16_t* v_cache;
    int prefix_cap, ring_cap, cache_cap;
    const int32_t* prefix_len;
    const int32_t* gen_index;
    const float* sink;
    float scale;
    double inv_freq[64];  // RoPE frequencies theta^(-2i/head_dim), i < head_dim/2 (host-computed)
    uint16_t* out;
    int64_t ld_out;
    int n_split;
    float* part;    // [rows][n_heads][n_split][head_dim + 2]
    uint16_t* k_scale;  // int8 caches: fp16 scale per (row, head, slot); NULL: fp16 caches
    uint16_t* v_scale;
};

// Prompt passes (prefill): n_seq sequences packed one after another (P
// positions in all), causal attention within each sequence.
constexpr int PREFILL_MAX_SEQ = 32;
struct PrefillAttnParams {
    int P, n_heads, head_dim;
    const float* qkv;    // [P][ld_qkv] fp32 projections (q | k | v)
    int64_t ld_qkv;
    uint16_t* q;         // [P][n_heads * head_dim] fp16 scratch: the rotated queries
    uint16_t* k_cache;   // the layer's caches [rows][n_heads][cache_cap][head_dim]; sequence s writes
    uint16_t* v_cache;   //   indices 0..len-1 of row seq_row[s]
    int cache_cap;
    float scale;
    double inv_freq[64];
    uint16_t* out;       // [P][ld_out] fp16 attention output
    int64_t ld_out;
    float* part;         // prefill_attn_part_bytes(...): partials of split windows
    int n_qb;            // query blocks of the longest sequence (set by the launcher)
    int n_seq;
    int seq_off[PREFILL_MAX_SEQ];  // first packed position of each sequence
    int seq_len[PREFILL_MAX_SEQ];
    int seq_row[PREFILL_MAX_SEQ];  // its cache row
    uint16_t* k_scale;   // INT8 caches: fp16 scales [rows][n_heads][cache_cap]; NULL: fp16 caches
    uint16_t* v_scale;
};

size_t prefill_attn_part_bytes(int n_seq, int max_len, int n_heads);
void prefill_set_rope(PrefillAttnParams& p, float theta);
void launch_attn_prefill(const PrefillAttnParams& p, hipStream_t s);

int attn_n_split(int cache_cap);
size_t attn_part_bytes(int rows, int n_heads, int head_dim, int cache_cap);
size_t attn_ws_bytes(int rows, int n_heads, int head_dim, int cache_cap);
void attn_set_rope(AttnParams& p, float theta);
void launch_attn(const AttnParams& p, hipStream_t s);
// Up to 16 rows with head_dim 128: the attention, then the merge of the
// splits fused with the O projection (W_o [n_out][n_heads * 128] in format
// fmt), added into the fixed-point residual h [rows][ldh] with atomic integer
// adds (order-independent).
bool attn_merge_o_ok(const AttnParams& p, int fmt, int n_out);
void launch_attn_merge_o(const AttnParams& p, int fmt, const uint8_t* wo, int n_out, fix_t* h, int64_t ldh,
                         uint32_t* status, hipStream_t s);
ocrdec_status check_attn(const ocrdec_attn_args* a);

}  // namespace ocrdec

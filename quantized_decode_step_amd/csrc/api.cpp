// Status plumbing, version, and the host-side packer (canonical blocks <->
// the tiled layout the kernels stream; see common.hpp for the layout).
#include <string.h>

#include <string>

#include "common.hpp"

namespace ocrdec {

static thread_local std::string g_last_error;

ocrdec_status fail(ocrdec_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

ocrdec_status ok() { return OCRDEC_OK; }

ocrdec_status launch_status(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OCRDEC_ERR_DEVICE, std::string(what) + ": " + hipGetErrorString(e));
    return OCRDEC_OK;
}

static thread_local ocrdec_profile* g_prof = nullptr;

void prof_mark(hipStream_t s, int kernel) {
    ocrdec_profile* p = g_prof;
    if (!p || p->count >= p->capacity) return;
    if (hipEventRecord((hipEvent_t)p->events[p->count], s) != hipSuccess) return;
    p->kernels[p->count] = kernel;
    p->count += 1;
}

ocrdec_status check_qmat(const ocrdec_qmat* w, const char* name) {
    if (!w) return fail(OCRDEC_ERR_INVALID_ARG, std::string(name) + ": NULL descriptor");
    PackGeom g;
    if (!pack_geom(w->fmt, &g)) return fail(OCRDEC_ERR_UNSUPPORTED, std::string(name) + ": unknown format");
    if (w->n <= 0 || w->k <= 0) return fail(OCRDEC_ERR_INVALID_ARG, std::string(name) + ": n and k must be positive");
    if (w->k % 32) return fail(OCRDEC_ERR_INVALID_ARG, std::string(name) + ": k must be a multiple of 32");
    if (!w->data) return fail(OCRDEC_ERR_INVALID_ARG, std::string(name) + ": NULL data");
    if ((uintptr_t)w->data & 255) return fail(OCRDEC_ERR_INVALID_ARG, std::string(name) + ": data not 256-byte aligned");
    return OCRDEC_OK;
}

// ---------------------------------------------------------------------------
// Packer
// ---------------------------------------------------------------------------

namespace {

inline uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
inline void wr16(uint8_t* p, uint16_t v) {
    p[0] = (uint8_t)(v & 255);
    p[1] = (uint8_t)(v >> 8);
}

int canon_block_bytes(int fmt) {
    switch (fmt) {
    case OCRDEC_Q8_0: return 34;
    case OCRDEC_Q4_0: return 18;
    case OCRDEC_U8A_G32: return 36;
    default: return 0;
    }
}

// Code of element i (0..31) of a canonical block.
inline int canon_code(int fmt, const uint8_t* blk, int i) {
    switch (fmt) {
    case OCRDEC_Q8_0: return (int)(int8_t)blk[2 + i];
    case OCRDEC_Q4_0: return i < 16 ? (blk[2 + i] & 15) : (blk[2 + i - 16] >> 4);
    case OCRDEC_U8A_G32: return blk[4 + i];
    default: return 0;
    }
}

inline void canon_set_code(int fmt, uint8_t* blk, int i, int q) {
    switch (fmt) {
    case OCRDEC_Q8_0: blk[2 + i] = (uint8_t)(int8_t)q; break;
    case OCRDEC_Q4_0:
        if (i < 16) blk[2 + i] = (uint8_t)((blk[2 + i] & 0xF0) | (q & 15));
        else blk[2 + i - 16] = (uint8_t)((blk[2 + i - 16] & 0x0F) | ((q & 15) << 4));
        break;
    case OCRDEC_U8A_G32: blk[4 + i] = (uint8_t)q; break;
    default: break;
    }
}

// Byte offset, inside a chunk's 1024 code bytes, of element i (0..7) of the
// 8-element run served to lane `lane` for block j of the chunk, and the bit
// shift inside that byte (Q4_0 only).
inline void code_pos(int fmt, int lane, int j, int i, int* byte, int* shift) {
    int base = lane * 16;
    switch (fmt) {
    case OCRDEC_F16: *byte = base + 2 * i; *shift = 0; break;
    case OCRDEC_Q8_0:
    case OCRDEC_U8A_G32: *byte = base + 8 * j + i; *shift = 0; break;
    case OCRDEC_Q4_0: {
        int p = i >> 1;
        int bit = (i & 1) ? 16 + 4 * p : 4 * p;
        *byte = base + 4 * j + (bit >> 3);
        *shift = bit & 7;
        break;
    }
    default: *byte = 0; *shift = 0;
    }
}

ocrdec_status check_pack_args(int32_t fmt, int32_t n, int32_t k) {
    PackGeom g;
    if (!pack_geom(fmt, &g)) return fail(OCRDEC_ERR_UNSUPPORTED, "unknown format");
    if (n <= 0 || k <= 0) return fail(OCRDEC_ERR_INVALID_ARG, "n and k must be positive");
    if (k % 32) return fail(OCRDEC_ERR_INVALID_ARG, "k must be a multiple of 32");
    return OCRDEC_OK;
}

}  // namespace
}  // namespace ocrdec

extern "C" ocrdec_status ocrdec_profile_set(ocrdec_profile* prof) {
    using namespace ocrdec;
    if (prof) {
        OCR_CHECK_ARG(prof->events && prof->kernels, "profile arrays must be non-NULL");
        OCR_CHECK_ARG(prof->capacity >= 0 && prof->count >= 0, "capacity and count must be >= 0");
    }
    g_prof = prof;
    return OCRDEC_OK;
}

extern "C" ocrdec_status ocrdec_profile_mark(void* stream) {
    using namespace ocrdec;
    ocrdec_profile* p = g_prof;
    if (!p || p->count >= p->capacity) return OCRDEC_OK;
    OCR_HIP(hipEventRecord((hipEvent_t)p->events[p->count], (hipStream_t)stream));
    p->kernels[p->count] = -1;
    p->count += 1;
    return OCRDEC_OK;
}

using namespace ocrdec;

extern "C" {

const char* ocrdec_last_error(void) { return g_last_error.c_str(); }

const char* ocrdec_version(void) { return "libocrdec 0.1 (gfx950)"; }

ocrdec_status ocrdec_packed_bytes(int32_t fmt, int32_t n, int32_t k, size_t* bytes) {
    ocrdec_status s = check_pack_args(fmt, n, k);
    if (s != OCRDEC_OK) return s;
    OCR_CHECK_ARG(bytes, "bytes is NULL");
    *bytes = packed_size(fmt, n, k);
    return OCRDEC_OK;
}

ocrdec_status ocrdec_pack(int32_t fmt, int32_t n, int32_t k, const void* canonical, void* packed) {
    ocrdec_status s = check_pack_args(fmt, n, k);
    if (s != OCRDEC_OK) return s;
    OCR_CHECK_ARG(canonical && packed, "NULL buffer");
    PackGeom g;
    pack_geom(fmt, &g);
    const uint8_t* src = (const uint8_t*)canonical;
    uint8_t* dst = (uint8_t*)packed;
    const int64_t T = n_tiles(n), C = n_chunks(fmt, k), nb = k / 32;
    memset(dst, 0, packed_size(fmt, n, k));
    const int cbb = canon_block_bytes(fmt);
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < C; ++c) {
            uint8_t* ch = dst + (t * C + c) * g.cb;
            // Q4_0 padding codes are 8 (value 0 even with a non-zero scale).
            if (fmt == OCRDEC_Q4_0) memset(ch, 0x88, 1024);
            for (int lane = 0; lane < 64; ++lane) {
                const int64_t row = t * 16 + (lane & 15);
                for (int j = 0; j < g.sb; ++j) {
                    const int64_t blk = c * g.sb + j;
                    if (row >= n || blk >= nb) continue;
                    for (int i = 0; i < 8; ++i) {
                        const int64_t col = blk * 32 + 8 * (lane >> 4) + i;
                        int byte, shift;
                        code_pos(fmt, lane, j, i, &byte, &shift);
                        if (fmt == OCRDEC_F16) {
                            memcpy(ch + byte, src + (row * k + col) * 2, 2);
                        } else if (fmt == OCRDEC_Q4_0) {
                            const uint8_t* b = src + (row * nb + blk) * cbb;
                            int q = canon_code(fmt, b, (int)(col - blk * 32));
                            ch[byte] = (uint8_t)((ch[byte] & ~(15 << shift)) | (q << shift));
                        } else {
                            const uint8_t* b = src + (row * nb + blk) * cbb;
                            ch[byte] = (uint8_t)canon_code(fmt, b, (int)(col - blk * 32));
                        }
                    }
                }
            }
            if (fmt == OCRDEC_F16) continue;
            for (int r = 0; r < 16; ++r) {
                const int64_t row = t * 16 + r;
                for (int j = 0; j < g.sb; ++j) {
                    const int64_t blk = c * g.sb + j;
                    if (row >= n || blk >= nb) continue;
                    const uint8_t* b = src + (row * nb + blk) * cbb;
                    uint8_t* sp = ch + 1024 + r * g.scb;
                    if (fmt == OCRDEC_U8A_G32) {
                        wr16(sp + 4 * j, rd16(b));
                        wr16(sp + 4 * j + 2, rd16(b + 2));
                    } else {
                        wr16(sp + 2 * j, rd16(b));
                    }
                }
            }
        }
    }
    return OCRDEC_OK;
}

ocrdec_status ocrdec_unpack(int32_t fmt, int32_t n, int32_t k, const void* packed, void* canonical) {
    ocrdec_status s = check_pack_args(fmt, n, k);
    if (s != OCRDEC_OK) return s;
    OCR_CHECK_ARG(canonical && packed, "NULL buffer");
    PackGeom g;
    pack_geom(fmt, &g);
    const uint8_t* src = (const uint8_t*)packed;
    uint8_t* dst = (uint8_t*)canonical;
    const int64_t C = n_chunks(fmt, k), nb = k / 32;
    const int cbb = canon_block_bytes(fmt);
    for (int64_t row = 0; row < n; ++row) {
        const int64_t t = row / 16;
        const int r = (int)(row % 16);
        for (int64_t blk = 0; blk < nb; ++blk) {
            const int64_t c = blk / g.sb;
            const int j = (int)(blk % g.sb);
            const uint8_t* ch = src + (t * C + c) * g.cb;
            uint8_t* b = (fmt == OCRDEC_F16) ? nullptr : dst + (row * nb + blk) * cbb;
            if (b) {
                const uint8_t* sp = ch + 1024 + r * g.scb;
                if (fmt == OCRDEC_U8A_G32) {
                    wr16(b, rd16(sp + 4 * j));
                    wr16(b + 2, rd16(sp + 4 * j + 2));
                } else {
                    wr16(b, rd16(sp + 2 * j));
                }
            }
            for (int e = 0; e < 32; ++e) {
                const int lane = r + 16 * (e >> 3);
                const int i = e & 7;
                int byte, shift;
                code_pos(fmt, lane, j, i, &byte, &shift);
                if (fmt == OCRDEC_F16) {
                    memcpy(dst + (row * k + blk * 32 + e) * 2, ch + byte, 2);
                } else if (fmt == OCRDEC_Q4_0) {
                    canon_set_code(fmt, b, e, (ch[byte] >> shift) & 15);
                } else if (fmt == OCRDEC_Q8_0) {
                    canon_set_code(fmt, b, e, (int)(int8_t)ch[byte]);
                } else {
                    canon_set_code(fmt, b, e, ch[byte]);
                }
            }
        }
    }
    return OCRDEC_OK;
}

}  // extern "C"

// Shared definitions of libocrdec: status plumbing, the packed weight layout,
// and device helpers for gfx950 (64-lane wavefronts, MFMA 16x16x32 f16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include <string>

#include "../../include/ocrdec.h"

namespace ocrdec {

// ---------------------------------------------------------------------------
// Status and messages (host)
// ---------------------------------------------------------------------------

ocrdec_status fail(ocrdec_status s, const std::string& msg);
ocrdec_status ok();

#define OCR_CHECK_ARG(cond, ...)                                                   \
    do {                                                                           \
        if (!(cond)) return ::ocrdec::fail(OCRDEC_ERR_INVALID_ARG, __VA_ARGS__);   \
    } while (0)

#define OCR_HIP(call)                                                              \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess)                                                      \
            return ::ocrdec::fail(OCRDEC_ERR_DEVICE,                               \
                                  std::string(#call) + ": " + hipGetErrorString(e_)); \
    } while (0)

// Checks the launch that was just enqueued.
ocrdec_status launch_status(const char* what);

// Records a profiling event before a kernel of kind `kernel` (ocrdec_kernel)
// if the calling thread has a profile set (ocrdec_profile_set).
void prof_mark(hipStream_t s, int kernel);

// ---------------------------------------------------------------------------
// Packed weight layout
//
// W[n][k] is cut into tiles of 16 output rows and chunks of KC input columns.
// Chunk (t, c) occupies CB bytes at offset (t * n_chunks + c) * CB:
//   bytes [0, 1024): the codes, 16 bytes per lane of a 64-lane wavefront.
//     Lane l serves row 16t + (l & 15) and the 8 consecutive columns
//     8*(l >> 4) .. +7 of every 32-column block of the chunk, which is the
//     B-operand layout of v_mfma_f32_16x16x32_f16 (column j = l & 15,
//     k = 8*(l >> 4) + i).  Block j of the chunk sits in
//       F16   the whole 16 bytes (8 halves), one block per chunk;
//       Q8_0  bytes 8j..8j+7 (int8), two blocks per chunk;
//       U8A   bytes 8j..8j+7 (uint8), two blocks per chunk;
//       Q4_0  dword j, four blocks per chunk; element 2p at bits 4p..4p+3 and
//             element 2p+1 at bits 16+4p..19+4p, so (dword >> 4p) & 0x000F000F
//             is a pair of codes in the two halves of a 32-bit register.
//   bytes [1024, CB): the scales of the 16 rows, row-major:
//       Q8_0  row r: fp16 d[block 0], d[block 1]              (4 bytes)
//       Q4_0  row r: fp16 d[block 0..3]                       (8 bytes)
//       U8A   row r: fp16 s0, z0, s1, z1                      (8 bytes)
// Rows >= n and blocks >= k/32 are zero.
// ---------------------------------------------------------------------------

struct PackGeom {
    int sb;     // 32-column blocks per chunk
    int kc;     // columns per chunk
    int cb;     // bytes per chunk
    int scb;    // scale bytes per row per chunk
};

inline bool pack_geom(int fmt, PackGeom* g) {
    switch (fmt) {
    case OCRDEC_F16: *g = {1, 32, 1024, 0}; return true;
    case OCRDEC_Q8_0: *g = {2, 64, 1088, 4}; return true;
    case OCRDEC_Q4_0: *g = {4, 128, 1152, 8}; return true;
    case OCRDEC_U8A_G32: *g = {2, 64, 1152, 8}; return true;
    default: return false;
    }
}

inline int64_t n_tiles(int n) { return (n + 15) / 16; }
inline int64_t n_chunks(int fmt, int k) {
    PackGeom g;
    pack_geom(fmt, &g);
    return (k + g.kc - 1) / g.kc;
}
inline size_t packed_size(int fmt, int n, int k) {
    PackGeom g;
    pack_geom(fmt, &g);
    size_t b = (size_t)n_tiles(n) * (size_t)n_chunks(fmt, k) * (size_t)g.cb;
    return (b + 255) & ~(size_t)255;
}

// Validates a device matrix descriptor.
ocrdec_status check_qmat(const ocrdec_qmat* w, const char* name);

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

// Bump allocator over a caller workspace.
struct Carve {
    char* base;
    size_t off = 0;
    explicit Carve(void* p) : base((char*)p) {}
    template <class T>
    T* take(size_t count) {
        T* p = (T*)(base ? base + off : nullptr);
        off += align256(count * sizeof(T));
        return p;
    }
};

}  // namespace ocrdec

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

typedef _Float16 f16_t;
typedef f16_t half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));  // 16 bytes in registers (arrays stay in VGPRs)
typedef f16_t half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

#define OCR_DEV __device__ __forceinline__

OCR_DEV float h2f(uint16_t h) { return (float)__builtin_bit_cast(f16_t, h); }
OCR_DEV uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, (f16_t)f); }

OCR_DEV float4v mfma16(half8v a, half8v b, float4v c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Sum over all 64 lanes (result in every lane).
// Wavefront reductions through DPP lane moves (VALU operations, no LDS round
// trip): quad swaps, half-row and row mirrors give every lane its 16-lane row
// total, two row broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2
// and 3) complete it in lane 63, which is returned to every lane.
template <int CTRL, int ROW_MASK = 0xF>
OCR_DEV float dpp_move(float v, float old) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                                 __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF,
                                                                 false));
}
OCR_DEV float lane63(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
OCR_DEV float wave_sum(float v) {
    v += dpp_move<0xB1>(v, 0.f);        // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v, 0.f);        // quad_perm [2,3,0,1]
    v += dpp_move<0x141>(v, 0.f);       // row_half_mirror
    v += dpp_move<0x140>(v, 0.f);       // row_mirror
    v += dpp_move<0x142, 0xA>(v, 0.f);  // row_bcast:15
    v += dpp_move<0x143, 0xC>(v, 0.f);  // row_bcast:31
    return lane63(v);
}
// Sum over each aligned group of W lanes (W = 4, 8 or 16), in every lane of
// the group: the first steps of wave_sum (DPP moves, no LDS permutes).
template <int W>
OCR_DEV float group_sum(float v) {
    static_assert(W == 4 || W == 8 || W == 16, "group width");
    v += dpp_move<0xB1>(v, 0.f);                          // quad_perm [1,0,3,2]
    v += dpp_move<0x4E>(v, 0.f);                          // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp_move<0x141>(v, 0.f);   // row_half_mirror
    if constexpr (W == 16) v += dpp_move<0x140>(v, 0.f);  // row_mirror
    return v;
}
// Bitwise OR over all 64 lanes (result in every lane), by the same DPP steps
// as wave_sum.
template <int CTRL, int ROW_MASK = 0xF>
OCR_DEV uint32_t dpp_move_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
}
OCR_DEV uint32_t wave_or(uint32_t v) {
    v |= dpp_move_u32<0xB1>(v);
    v |= dpp_move_u32<0x4E>(v);
    v |= dpp_move_u32<0x141>(v);
    v |= dpp_move_u32<0x140>(v);
    v |= dpp_move_u32<0x142, 0xA>(v);
    v |= dpp_move_u32<0x143, 0xC>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}
OCR_DEV unsigned long long wave_or(unsigned long long v) {
    return (unsigned long long)wave_or((uint32_t)v) | ((unsigned long long)wave_or((uint32_t)(v >> 32)) << 32);
}
OCR_DEV float wave_max(float v) {
    v = fmaxf(v, dpp_move<0xB1>(v, v));
    v = fmaxf(v, dpp_move<0x4E>(v, v));
    v = fmaxf(v, dpp_move<0x141>(v, v));
    v = fmaxf(v, dpp_move<0x140>(v, v));
    v = fmaxf(v, dpp_move<0x142, 0xA>(v, v));
    v = fmaxf(v, dpp_move<0x143, 0xC>(v, v));
    return lane63(v);
}

OCR_DEV half8v bits_to_half8(uint4 q) { return __builtin_bit_cast(half8v, q); }

OCR_DEV half2v u32_to_h2(uint32_t u) { return __builtin_bit_cast(half2v, u); }
OCR_DEV uint32_t h2_to_u32(half2v h) { return __builtin_bit_cast(uint32_t, h); }

// (x & m) | c for a constant c with no bits in m, in one VALU operation
// (v_and_or_b32).  With both m and c literals the compiler emits a separate
// and + or; an empty asm statement hides c's value, so it is kept in a
// register and the three-operand form applies.  The asm emits no instruction:
// the hardware's register-dependency rules stay with the compiler.
OCR_DEV uint32_t mask_or(uint32_t x, uint32_t m, uint32_t c) {
    asm("" : "+v"(c));
    return (x & m) | c;
}

// Eight Q4_0 codes (one packed dword) -> the eight fp16 values q - 8 (exact).
OCR_DEV half8v deq_q4(uint32_t dw) {
    const half2v off = {(f16_t)1032.0f, (f16_t)1032.0f};
    constexpr uint32_t M = 0x000F000Fu, E = 0x64006400u;
    half2v p0 = u32_to_h2(mask_or(dw, M, E)) - off;
    half2v p1 = u32_to_h2(mask_or(dw >> 4, M, E)) - off;
    half2v p2 = u32_to_h2(mask_or(dw >> 8, M, E)) - off;
    half2v p3 = u32_to_h2(mask_or(dw >> 12, M, E)) - off;
    uint4 r = {h2_to_u32(p0), h2_to_u32(p1), h2_to_u32(p2), h2_to_u32(p3)};
    return bits_to_half8(r);
}

// Eight Q4_0 codes (one packed dword) -> their raw nibbles n_i = q_i + 8 as
// fp16 subnormals, n_i * 2^-24 exactly (the matrix cores take subnormal fp16
// operands at their value): four masks and three shifts, no conversion.  The
// products with fp16 activations are exact in fp32; the offset 8 and the
// factor 2^-24 are taken out through the accumulator (q4_bias, Q4_RAW_SCALE).
OCR_DEV half8v deq_q4_raw(uint32_t dw) {
    constexpr uint32_t M = 0x000F000Fu;
    uint4 r = {dw & M, (dw >> 4) & M, (dw >> 8) & M, (dw >> 12) & M};
    return bits_to_half8(r);
}
constexpr float Q4_RAW_SCALE = 16777216.0f;  // 2^24

// The same codes with one shift per dword: positions 0, 1, 4, 5 hold
// n * 2^-24 and positions 2, 3, 6, 7 (nibbles left at bits 4-7) hold
// 16 n * 2^-24, for activations whose positions 2, 3, 6, 7 were divided by 16
// (q4_split_prepare), which makes every product x n 2^-24 again.
OCR_DEV half8v deq_q4_split(uint32_t dw) {
    constexpr uint32_t M0 = 0x000F000Fu, M1 = 0x00F000F0u;
    const uint32_t h = dw >> 8;
    uint4 r = {dw & M0, dw & M1, h & M0, h & M1};
    return bits_to_half8(r);
}

// Eight int8 codes (two dwords, k order) -> fp16 q (exact).  1024 + (q ^ 0x80)
// is built with a byte permute against 0x64 and 1152 is subtracted.
OCR_DEV half8v deq_q8(uint32_t lo, uint32_t hi) {
    const half2v off = {(f16_t)1152.0f, (f16_t)1152.0f};
    uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
    half2v p0 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, a, 0x04010400u)) - off;
    half2v p1 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, a, 0x04030402u)) - off;
    half2v p2 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04010400u)) - off;
    half2v p3 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, b, 0x04030402u)) - off;
    uint4 r = {h2_to_u32(p0), h2_to_u32(p1), h2_to_u32(p2), h2_to_u32(p3)};
    return bits_to_half8(r);
}

// Eight uint8 codes -> fp16 q (exact).
OCR_DEV half8v deq_u8(uint32_t lo, uint32_t hi) {
    const half2v off = {(f16_t)1024.0f, (f16_t)1024.0f};
    half2v p0 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u)) - off;
    half2v p1 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u)) - off;
    half2v p2 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u)) - off;
    half2v p3 = u32_to_h2(__builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)) - off;
    uint4 r = {h2_to_u32(p0), h2_to_u32(p1), h2_to_u32(p2), h2_to_u32(p3)};
    return bits_to_half8(r);
}

OCR_DEV float silu(float z) { return z / (1.0f + __expf(-z)); }

// ---------------------------------------------------------------------------
// The decode step's residual stream in exact fixed point
//
// h is held as int64 with 32 fraction bits.  Every addend (an fp32 projection
// output) is converted once, rounded to the nearest multiple of 2^-32, and
// the sums are integer sums: exact and independent of the order in which
// workgroups add their parts (atomic adds included), so the step is bitwise
// reproducible.  The range is |h| < 2^30; a non-finite addend or one beyond
// the range is replaced by 0 and reported through the status word.  Readers
// convert to fp32.
// ---------------------------------------------------------------------------

typedef long long fix_t;
constexpr float kFixLimit = 1073741824.0f;  // 2^30

// Status word bits (the decode step's workspace; ocrdec_device_status).
constexpr uint32_t kStatTokenRange = 1u, kStatResidual = 2u, kStatLogit = 4u, kStatNoToken = 8u;

// a = fl + f with fl = floor(a) (an integer below 2^30 in magnitude) and f in
// [0, 1) exact in fp32; f * 2^32 is an integer whenever |a| >= 2^-9 and is
// rounded to the nearest one below that, so the conversion is exact except
// for the bits of tiny addends below 2^-32.  All in fp32/int32 arithmetic.
OCR_DEV fix_t fix_from(float a, bool& bad) {
    const bool ok = fabsf(a) < kFixLimit;  // false for NaN
    bad |= !ok;
    a = ok ? a : 0.f;
    const float fl = floorf(a);
    const uint32_t lo = (uint32_t)rintf((a - fl) * 4294967296.0f);  // <= 2^32 - 2^8
    return (fix_t)(((uint64_t)(uint32_t)(int32_t)fl << 32) | lo);
}
// hi + lo * 2^-32 with one fused rounding (hi exact below 2^24).
OCR_DEV float fix_to(fix_t v) {
    return fmaf((float)(uint32_t)v, 2.3283064365386963e-10f, (float)(int32_t)(v >> 32));
}

// Four consecutive residual values (fp32 or fixed point) at index 4*c4.
OCR_DEV float4 ld_resid4(const float* h, int c4) { return ((const float4*)h)[c4]; }
OCR_DEV float4 ld_resid4(const fix_t* h, int c4) {
    const longlong2 a = ((const longlong2*)h)[2 * c4], b = ((const longlong2*)h)[2 * c4 + 1];
    return make_float4(fix_to(a.x), fix_to(a.y), fix_to(b.x), fix_to(b.y));
}
// Stores four values at index 4*c4 and returns them as a reader will load them.
OCR_DEV float4 st_resid4(float* h, int c4, float4 v, bool&) {
    ((float4*)h)[c4] = v;
    return v;
}
OCR_DEV float4 st_resid4(fix_t* h, int c4, float4 v, bool& bad) {
    const fix_t a = fix_from(v.x, bad), b = fix_from(v.y, bad), c = fix_from(v.z, bad), d = fix_from(v.w, bad);
    ((longlong2*)h)[2 * c4] = make_longlong2(a, b);
    ((longlong2*)h)[2 * c4 + 1] = make_longlong2(c, d);
    return make_float4(fix_to(a), fix_to(b), fix_to(c), fix_to(d));
}

// The status area of the decode step's workspace: word 0 collects the bits
// the step's kernels raise with atomic ORs; word 1 + r holds row r's input
// bits, written by the first kernel, which also clears word 0 and the words
// of rows past the batch (up to kStatusRows).  Later kernels run after it in
// stream order, so nothing is lost to the clearing.
constexpr int kStatusRows = 32;
OCR_DEV void status_begin(uint32_t* status, int r, int rows, bool tok_bad, bool resid_bad) {
    if (!status) return;
    const int lane = threadIdx.x & 63;
    const bool rb = __ballot(resid_bad) != 0;
    if (lane == 0) status[1 + r] = (tok_bad ? kStatTokenRange : 0u) | (rb ? kStatResidual : 0u);
    if (r == 0) {
        if (lane == 0) status[0] = 0;
        if (lane >= rows && lane < kStatusRows) status[1 + lane] = 0;
    }
}

// h[i] += a as an atomic integer add (any order gives the same sum).
OCR_DEV void fix_atomic_add(fix_t* h, float a, bool& bad) {
    atomicAdd((unsigned long long*)h, (unsigned long long)fix_from(a, bad));
}

// Sets `bits` in the status word if any lane of the wavefront raised `flag`
// (one atomic per wavefront).
OCR_DEV void report_status(uint32_t* status, bool flag, uint32_t bits) {
    const unsigned long long m = __ballot(flag);
    if (status && m && (threadIdx.x & 63) == (unsigned)__builtin_ctzll(m)) atomicOr(status, bits);
}

// The four-value groups c4 = lane + 64 i (i < NV) of one residual row of H
// values (H % 4 == 0, n4 = H / 4 groups) as fp32, zero past the row.  Every
// load is issued before the first use (addresses clamped into the row, no
// branches), so the row costs one memory round trip in either form.
template <int NV>
OCR_DEV void load_resid_row(const float* h, int n4, float4 (&v)[NV]) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = ((const float4*)h)[min(lane + 64 * i, n4 - 1)];
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (lane + 64 * i >= n4) v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}
template <int NV>
OCR_DEV void load_resid_row(const fix_t* h, int n4, float4 (&v)[NV]) {
    const int lane = threadIdx.x & 63;
    longlong2 a[NV], b[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c = min(lane + 64 * i, n4 - 1);
        a[i] = ((const longlong2*)h)[2 * c];
        b[i] = ((const longlong2*)h)[2 * c + 1];
    }
#pragma unroll
    for (int i = 0; i < NV; ++i)
        v[i] = lane + 64 * i < n4 ? make_float4(fix_to(a[i].x), fix_to(a[i].y), fix_to(b[i].x), fix_to(b[i].y))
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
}

// x = fp16(v / sqrt(mean(v^2) + eps) * gamma) for one row held in registers
// as load_resid_row leaves it (one wavefront).  The gains are requested first.
// The result goes to x and to xl (LDS), each if non-NULL.
template <int NV>
OCR_DEV void rmsnorm_regs(const float4 (&v)[NV], const uint16_t* gamma, int H, float eps, uint16_t* x,
                          uint16_t* xl) {
    const int lane = threadIdx.x & 63;
    const int n4 = H / 4;
    uint2 g[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) g[i] = ((const uint2*)gamma)[min(lane + 64 * i, n4 - 1)];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
    ss = wave_sum(ss);
    const float inv = 1.0f / sqrtf(ss / (float)H + eps);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int c4 = lane + 64 * i;
        if (c4 < n4) {
            const uint32_t lo = (uint32_t)f2h(v[i].x * inv * h2f((uint16_t)(g[i].x & 0xFFFF))) |
                                ((uint32_t)f2h(v[i].y * inv * h2f((uint16_t)(g[i].x >> 16))) << 16);
            const uint32_t hi = (uint32_t)f2h(v[i].z * inv * h2f((uint16_t)(g[i].y & 0xFFFF))) |
                                ((uint32_t)f2h(v[i].w * inv * h2f((uint16_t)(g[i].y >> 16))) << 16);
            if (x) ((uint2*)x)[c4] = make_uint2(lo, hi);
            if (xl) ((uint2*)xl)[c4] = make_uint2(lo, hi);
        }
    }
}

// x = fp16(h / sqrt(mean(h^2) + eps) * gamma) for one residual row (fp32 or
// fixed point) of H <= 256 * NV values (H % 4 == 0) by one wavefront: one
// memory round trip for the row and the gains.
template <int NV = 16, class HT = float>
OCR_DEV void wave_rmsnorm_row(const HT* h, const uint16_t* gamma, int H, float eps, uint16_t* x,
                              uint16_t* xl = nullptr) {
    float4 v[NV];
    load_resid_row<NV>(h, H / 4, v);
    rmsnorm_regs<NV>(v, gamma, H, eps, x, xl);
}

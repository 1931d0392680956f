// common.h -- internal definitions shared by the HIP kernels and the C ABI.
//
// Method: "UltraSketchLLM: Sub-1-Bit LLM Compression via Sketch and
// Hardware-Friendly Operators" (gist.science explainer, "Resumen Técnico",
// Metodología §1, §2, §4).  Only gfx950 (MI355X) is targeted.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/sketch.h"

namespace sketch {

// ---------------------------------------------------------------------------
// Projection buffer layout (index form of the one-hot projection P).
// Every section starts on a 256-byte boundary.
//   header : ProjHeader
//   idx    : uint16[R*N]        forward map k(l), l = r*N + j
//   off    : uint32[R*Bg + 1]   CSR offsets of the inverse map, row-major (r, k)
//   cols   : uint16[R*N]        columns j of every (r, k) segment, ascending
//   cnt    : uint32[R*Bg]       build scratch (per-segment counters)
// ---------------------------------------------------------------------------
constexpr uint32_t kProjMagic = 0x31504B53u;      // "SKP1"
constexpr uint32_t kProjMagicRows = 0x32504B53u;  // "SKP2": multi-row sketch, rows in pad[0]
constexpr uint32_t kProjMagicHash = 0x33504B53u;  // "SKP3": allocated sketch, 32-bit hash per local index
constexpr uint32_t kProjVersion = 1;

struct ProjHeader {
    uint32_t magic, version, R, N, Bg, seed, pad[2];
};
static_assert(sizeof(ProjHeader) == 32, "kernels read the header as two 16-byte vectors");

struct ProjLayout {
    size_t idx, off, cols, cnt, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline ProjLayout proj_layout(int64_t R, int64_t N, int64_t Bg) {
    ProjLayout L;
    size_t at = align256(sizeof(ProjHeader));
    L.idx = at;
    at = align256(at + sizeof(uint16_t) * size_t(R * N));
    L.off = at;
    at = align256(at + sizeof(uint32_t) * size_t(R * Bg + 1));
    L.cols = at;
    at = align256(at + sizeof(uint16_t) * size_t(R * N));
    L.cnt = at;
    at = align256(at + sizeof(uint32_t) * size_t(R * Bg));
    L.total = at;
    return L;
}

// Projection of an allocated sketch: header, then H[l] = fmix32((l *
// 0x9E3779B1) ^ seed) for l < R*N (uint32); block b's bucket of l is
// umulhi(H[l], Bg_b).
inline ProjLayout proj_layout_hash(int64_t R, int64_t N) {
    ProjLayout L{};
    L.idx = align256(sizeof(ProjHeader));
    L.total = align256(L.idx + sizeof(uint32_t) * size_t(R * N));
    L.off = L.cols = L.cnt = L.total;
    return L;
}

// Validated shape of one call.
struct Shape {
    int64_t M, N, R, Bg, nb;
    int64_t rows;            // sketch rows (1: the single-row sketch)
    const uint32_t* boff;    // allocation: table offsets [nb + 1] (device), or nullptr
    int64_t bg_max;          // allocation: largest block count
    int64_t bits;            // bucket width: 16 (binary16) or 4 (codes + per-block scales)
};

// Checks the parameters of one call (the rules of sketch_layout) and fills
// the shape; defined with the C ABI.
sketch_status validate_params(const sketch_params* p, Shape* s);

// 4-bit buckets: byte offset of the block scales inside the tables buffer.
inline size_t q4_scales_offset(const Shape& s) { return align256(size_t(s.nb) * size_t(s.Bg / 2)); }

// Block b of an allocated sketch: its table offset and count, or false when
// the offsets are out of range (count 0 or above bg_max, or past the
// uniform budget nb * Bg that the tables were sized for).
__device__ inline bool alloc_block(const uint32_t* boff, int64_t b, uint32_t bg_max, uint64_t total, uint32_t& off,
                                   uint32_t& cnt) {
    const uint32_t o0 = boff[b], o1 = boff[b + 1];
    off = o0;
    cnt = o1 - o0;
    return o1 > o0 && cnt <= bg_max && uint64_t(o1) <= total;
}

// ---------------------------------------------------------------------------
// Bucket hash.  k(l) = (u64(fmix32((u32)(l * 0x9E3779B1) ^ seed)) * Bg) >> 32
// fmix32 is MurmurHash3's 32-bit finalizer (xor-shift / multiply rounds).
// ---------------------------------------------------------------------------
__host__ __device__ inline uint32_t fmix32(uint32_t h) {
    h ^= h >> 16;
    h *= 0x85EBCA6Bu;
    h ^= h >> 13;
    h *= 0xC2B2AE35u;
    h ^= h >> 16;
    return h;
}

__host__ __device__ inline uint32_t bucket_of(uint32_t l, uint32_t seed, uint32_t Bg) {
    uint32_t h = fmix32((l * 0x9E3779B1u) ^ seed);
    return uint32_t((uint64_t(h) * Bg) >> 32);
}

// ---------------------------------------------------------------------------
// Element loads widened to float (exact for all three formats).
// ---------------------------------------------------------------------------
__device__ inline float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ inline float f16_bits_to_f32(uint32_t h16) {
    _Float16 h;
    uint16_t v = uint16_t(h16);
    __builtin_memcpy(&h, &v, 2);
    return float(h);
}

template <int DT>
__device__ inline float load_elem(const void* base, int64_t e) {
    if constexpr (DT == SKETCH_F32) {
        return static_cast<const float*>(base)[e];
    } else if constexpr (DT == SKETCH_BF16) {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[e]);
    } else {
        return f16_bits_to_f32(static_cast<const uint16_t*>(base)[e]);
    }
}

// Same with a 32-bit element index (lets the compiler address off a uniform
// base with 32-bit per-lane offsets).
template <int DT>
__device__ inline float load_elem32(const void* base, uint32_t e) {
    if constexpr (DT == SKETCH_F32) {
        return static_cast<const float*>(base)[e];
    } else if constexpr (DT == SKETCH_BF16) {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[e]);
    } else {
        return f16_bits_to_f32(static_cast<const uint16_t*>(base)[e]);
    }
}

// float -> binary16 bits, round to nearest even (v_cvt_f16_f32 in the
// default rounding mode; binary16 denormals are kept on gfx9).
__device__ inline uint16_t f32_to_f16_bits(float f) {
    _Float16 h = static_cast<_Float16>(f);
    uint16_t v;
    __builtin_memcpy(&v, &h, 2);
    return v;
}

typedef uint32_t vec4u32 __attribute__((ext_vector_type(4)));

// 8 consecutive elements (e0 .. e0+7, 16- or 32-byte aligned) widened to float.
template <int DT>
__device__ inline void load8_f32(const void* base, int64_t e0, float (&f)[8]) {
    if constexpr (DT == SKETCH_F32) {
        const vec4u32* p = reinterpret_cast<const vec4u32*>(static_cast<const float*>(base) + e0);
        const vec4u32 u = p[0], v = p[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = __uint_as_float(u[e]);
            f[4 + e] = __uint_as_float(v[e]);
        }
    } else {
        const vec4u32 v = *reinterpret_cast<const vec4u32*>(static_cast<const uint16_t*>(base) + e0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h = (v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
            f[e] = DT == SKETCH_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
        }
    }
}

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ inline uint32_t f32_to_bf16_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Decoded weights out: W_hat element(s) of output dtype OD, from binary16
// bucket bits (binary16: the bits; float32: exact; bfloat16: rounded to
// nearest even) ...
template <int OD>
__device__ inline void store1_bits(void* out, int64_t e, uint32_t h) {
    if constexpr (OD == SKETCH_F32)
        static_cast<float*>(out)[e] = f16_bits_to_f32(h);
    else
        static_cast<uint16_t*>(out)[e] = uint16_t(OD == SKETCH_BF16 ? f32_to_bf16_bits(f16_bits_to_f32(h)) : h);
}

// The 8-element stores below are non-temporal: a materialised W_hat is
// written once and not read again by the kernel, and streaming it past the
// caches measured 12.1 -> 9.1 us for a 32 MiB bfloat16 decode.
typedef float vec4f32 __attribute__((ext_vector_type(4)));

template <int OD>
__device__ inline void store8_bits(void* out, int64_t e0, const uint32_t (&h)[8]) {
    if constexpr (OD == SKETCH_F32) {
        vec4f32* p = reinterpret_cast<vec4f32*>(static_cast<float*>(out) + e0);
        __builtin_nontemporal_store(vec4f32{f16_bits_to_f32(h[0]), f16_bits_to_f32(h[1]), f16_bits_to_f32(h[2]),
                                            f16_bits_to_f32(h[3])}, p);
        __builtin_nontemporal_store(vec4f32{f16_bits_to_f32(h[4]), f16_bits_to_f32(h[5]), f16_bits_to_f32(h[6]),
                                            f16_bits_to_f32(h[7])}, p + 1);
    } else {
        uint32_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = OD == SKETCH_BF16 ? f32_to_bf16_bits(f16_bits_to_f32(h[e])) : h[e];
        __builtin_nontemporal_store(
            vec4u32{v[0] | (v[1] << 16), v[2] | (v[3] << 16), v[4] | (v[5] << 16), v[6] | (v[7] << 16)},
            reinterpret_cast<vec4u32*>(static_cast<uint16_t*>(out) + e0));
    }
}

// ... or from float values (binary16 and bfloat16 rounded to nearest even).
template <int OD>
__device__ inline void store1_val(void* out, int64_t e, float v) {
    if constexpr (OD == SKETCH_F32)
        static_cast<float*>(out)[e] = v;
    else
        static_cast<uint16_t*>(out)[e] = uint16_t(OD == SKETCH_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
}

template <int OD>
__device__ inline void store8_val(void* out, int64_t e0, const float (&v)[8]) {
    if constexpr (OD == SKETCH_F32) {
        vec4f32* p = reinterpret_cast<vec4f32*>(static_cast<float*>(out) + e0);
        __builtin_nontemporal_store(vec4f32{v[0], v[1], v[2], v[3]}, p);
        __builtin_nontemporal_store(vec4f32{v[4], v[5], v[6], v[7]}, p + 1);
    } else {
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = OD == SKETCH_BF16 ? f32_to_bf16_bits(v[e]) : f32_to_f16_bits(v[e]);
        __builtin_nontemporal_store(
            vec4u32{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)},
            reinterpret_cast<vec4u32*>(static_cast<uint16_t*>(out) + e0));
    }
}

// ---------------------------------------------------------------------------
// Launch helpers (host side), defined in the .hip translation units.
// ---------------------------------------------------------------------------
sketch_status launch_projection_build(const sketch_params* p, const Shape& s, void* proj,
                                      hipStream_t stream);
// Writes the header, the last launch of every projection build.
sketch_status launch_proj_header(void* proj, const ProjHeader& h, hipStream_t stream);
sketch_status launch_encode(const sketch_params* p, const Shape& s, const void* proj, const void* W,
                            const float* imp, uint16_t* tables, int32_t* status, hipStream_t stream);
// The same with a library-held status word, then a wait for the stream and
// the flags as a status (sketch_encode with status_dev == NULL).
sketch_status launch_encode_sync(const sketch_params* p, const Shape& s, const void* proj, const void* W,
                                 const float* imp, uint16_t* tables, hipStream_t stream);
size_t gemv_workspace_bytes(const Shape& s, int64_t batch, sketch_dtype xdt);
sketch_status launch_gemv(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                          const void* X, sketch_dtype xdt, int64_t batch, float* Y, void* ws,
                          hipStream_t stream);
bool gemm_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch);
sketch_status launch_gemm(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                          const void* X, int64_t batch, float* Y, hipStream_t stream);

sketch_status launch_decode(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                            void* out, sketch_dtype out_dtype, hipStream_t stream);
sketch_status launch_decode_hashed(const sketch_params* p, const Shape& s, const uint16_t* tables, void* out,
                                   sketch_dtype out_dtype, hipStream_t stream);

// Multi-row sketch (rows.hip).
ProjLayout proj_layout_rows(int64_t R, int64_t N, int64_t rows);
sketch_status launch_projection_build_rows(const sketch_params* p, const Shape& s, void* proj, hipStream_t stream);
bool gemm_rows_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch);
// ws: optional; with rows_gemm_split_bytes(...) bytes the prefill product
// splits K over more workgroups
sketch_status launch_matmul_rows(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                                 const void* X, sketch_dtype xdt, int64_t batch, float* Y, void* ws, size_t ws_bytes,
                                 hipStream_t stream);
size_t rows_gemm_split_bytes(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch);
// The part of sketch_workspace_bytes a call cannot do without (the rest
// only speeds the call up).
sketch_status required_workspace_bytes(const sketch_params* p, int64_t batch, sketch_dtype x_dtype, size_t* bytes);

// Importance-aware allocation (alloc.hip).
sketch_status launch_projection_build_hash(const sketch_params* p, const Shape& s, void* proj, hipStream_t stream);
sketch_status launch_block_importance(const sketch_params* p, const Shape& s, const void* W, const float* a2,
                                      float* scores, hipStream_t stream);
bool gemm_alloc_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch);
sketch_status launch_matmul_alloc(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                                  const void* X, sketch_dtype xdt, int64_t batch, float* Y, hipStream_t stream);
sketch_status launch_decode_alloc(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                                  void* out, sketch_dtype out_dtype, bool hashed, hipStream_t stream);

// 4-bit buckets (q4.hip; the prefill product of the matrix-core tile kernel in gemm.hip).
bool gemm_tile_q4_supported(const Shape& s, sketch_dtype xdt, int64_t batch);
sketch_status launch_gemm_tile_q4(const sketch_params* p, const Shape& s, const void* proj, const uint8_t* codes,
                                  const uint16_t* scales, const void* X, int64_t batch, float* Y, hipStream_t stream);
sketch_status launch_matmul_q4(const sketch_params* p, const Shape& s, const void* proj, const void* tables,
                               const void* X, sketch_dtype xdt, int64_t batch, float* Y, hipStream_t stream);
sketch_status launch_decode_q4(const sketch_params* p, const Shape& s, const void* proj, const void* tables,
                               void* out, sketch_dtype out_dtype, bool hashed, hipStream_t stream);

inline sketch_status launch_status() {
    return hipGetLastError() == hipSuccess ? SKETCH_OK : SKETCH_EDEVICE;
}

}  // namespace sketch

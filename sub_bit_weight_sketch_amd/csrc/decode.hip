// decode.hip -- materialising W_hat = S * P^T (decompression).
//
// "Resumen Técnico" › Metodología §4: decompression is the matrix product
// W_hat = S * P^T; with P one-hot and shared by every row block this is
//     W_hat[i][j] = S[i / R][k((i % R) * N + j)].
// "Resumen Técnico" › Resultados Experimentales › Latencia de Sobrecarga
// compares that matrix form with a naive hash-based sketch, which hashes
// every weight and reads its bucket wherever it lies; decode_hashed_kernel is
// that baseline, kept to measure the ratio on this part.
//
// Multi-row sketch (Metodología §1: several hash functions, a sketch row
// each, the Max over the rows at decompression): the projection holds one
// forward map per row and W_hat[i][j] is, among the rows' buckets, the one of
// largest magnitude (AbsMin; smallest for AbsMax), the first row on ties.
// The kernels below take the row count at run time; MR selects the pick.
//
// decode_map_kernel: HBM-write-bound.  A workgroup stages the tables of GB
// consecutive row blocks in LDS and sweeps a span of columns of all R rows:
// per 8 columns of one row it loads the 16-byte slice of the forward map
// once (shared by every block, cache-resident) and, for each of its GB
// blocks, gathers 8 buckets from LDS and writes 8 outputs with one store.
#include "common.h"

namespace sketch {
namespace {

constexpr int kDecThreads = 256;
constexpr size_t kDecTableLds = 8 * 1024;    // tables of one workgroup (at least one table)
constexpr int kDecMaxGroup = 16;             // blocks per workgroup

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DecArgs {
    const uint16_t* S;     // [nb][Bg] binary16
    const uint16_t* idx;   // forward map [R*N] (map kernel only)
    const ProjHeader* hdr; // (map kernel only)
    void* out;             // [M][N] of the output dtype
    int64_t M, N, nb;
    uint32_t R, Bg, seed;
    uint32_t rows;         // sketch rows (forward maps idx[rho * R * N + l]; buckets of row rho hashed over Bg / rows)
    uint32_t GB;           // blocks per workgroup
    uint32_t nbg;          // block groups
    uint32_t span;         // columns per workgroup (a multiple of 8 on the vector path)
};

// Candidate v of a later sketch row replaces the kept bucket h (magnitude m)
// when strictly larger in magnitude (AbsMin) or strictly smaller (AbsMax); a
// NaN never replaces and is never replaced.
template <int RULE>
__device__ inline void keep(uint32_t& h, float& m, uint32_t v) {
    const float f = __builtin_fabsf(f16_bits_to_f32(v));
    if (RULE == SKETCH_ABSMIN ? f > m : f < m) {
        h = v;
        m = f;
    }
}

// Multi-row picks of 8 consecutive positions for Q consecutive staged
// tables g .. g+Q-1; map points at row 0's forward-map slice of the 8
// positions, L = R * N apart per row.
template <int RULE, int Q>
__device__ inline void pick_blocks(const uint16_t* tabs, uint32_t Bg, uint32_t g, const uint16_t* map, int64_t L,
                                   uint32_t rows, uint32_t (&h)[Q][8]) {
    float m[Q][8];
    // the first two rows' slices go out together (a multi-row sketch has at
    // least two); further rows load in the loop
    const u32x4 kv0 = *reinterpret_cast<const u32x4*>(map);
    const u32x4 kv1 = *reinterpret_cast<const u32x4*>(map + (rows > 1 ? L : 0));
    for (uint32_t rho = 0; rho < rows; ++rho) {
        const u32x4 kv = rho == 0 ? kv0 : rho == 1 ? kv1 : *reinterpret_cast<const u32x4*>(map + int64_t(rho) * L);
        const uint32_t ks[8] = {kv.x & 0xFFFFu, kv.x >> 16, kv.y & 0xFFFFu, kv.y >> 16,
                                kv.z & 0xFFFFu, kv.z >> 16, kv.w & 0xFFFFu, kv.w >> 16};
        uint32_t ka[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ka[e] = ks[e] < Bg ? ks[e] : 0;
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t v = tabs[(g + q) * Bg + ka[e]];
                if (rho == 0) {
                    h[q][e] = v;
                    m[q][e] = __builtin_fabsf(f16_bits_to_f32(v));
                } else {
                    keep<RULE>(h[q][e], m[q][e], v);
                }
            }
    }
}

__device__ inline bool map_header_ok(const ProjHeader* h, const DecArgs& a) {
    const bool magic = a.rows == 1 ? h->magic == kProjMagic : (h->magic == kProjMagicRows && h->pad[0] == a.rows);
    return magic && h->version == kProjVersion && h->R == a.R && h->N == uint32_t(a.N) && h->Bg == a.Bg &&
           h->seed == a.seed;
}

// VEC: N % 8 == 0 (16-byte forward-map slices and output rows).
// MR: multi-row sketch with the pick of rule RULE.
template <int OD, bool VEC, bool MR, int RULE>
__global__ __launch_bounds__(kDecThreads) void decode_map_kernel(DecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t tabs[];   // [GB][Bg]
    const uint32_t bg = blockIdx.x % a.nbg, sp = blockIdx.x / a.nbg;
    const int64_t b0 = int64_t(bg) * a.GB;
    const uint32_t gb = uint32_t(a.nb - b0 < int64_t(a.GB) ? a.nb - b0 : a.GB);
    const int64_t j0 = int64_t(sp) * a.span;
    const int64_t j1 = j0 + a.span < a.N ? j0 + a.span : a.N;
    const bool ok = map_header_ok(a.hdr, a);

    // tables of the group's blocks (contiguous in memory) -> LDS
    const uint32_t words = gb * a.Bg;   // binary16 entries
    const uint16_t* src = a.S + b0 * a.Bg;
    for (uint32_t e = threadIdx.x * 8; e < words; e += kDecThreads * 8) {
        if (e + 8 <= words && ((reinterpret_cast<uintptr_t>(src + e) & 15) == 0)) {
            *reinterpret_cast<u32x4*>(tabs + e) = *reinterpret_cast<const u32x4*>(src + e);
        } else {
            for (uint32_t q = e; q < words && q < e + 8; ++q) tabs[q] = src[q];
        }
    }
    __syncthreads();

    // A projection built for other parameters gives NaN everywhere (a
    // binary16 quiet NaN, which every output dtype turns into its own NaN)
    // and its forward map is not read at all.
    constexpr uint32_t kNaN16 = 0x7E00u;
    if (!ok) {
        const uint32_t w = uint32_t(j1 - j0);
        for (uint32_t u = threadIdx.x; u < a.R * w; u += kDecThreads)
            for (uint32_t g = 0; g < gb; ++g)
                store1_bits<OD>(a.out, ((b0 + g) * a.R + u / w) * a.N + j0 + (u % w), kNaN16);
        return;
    }
    if constexpr (MR) {
        const int64_t L = int64_t(a.R) * a.N;
        if constexpr (VEC) {
            const uint32_t cpr = uint32_t((j1 - j0) / 8);
            for (uint32_t u = threadIdx.x; u < a.R * cpr; u += kDecThreads) {
                const uint32_t r = u / cpr;
                const int64_t j = j0 + int64_t(u % cpr) * 8;
                const uint16_t* map = a.idx + int64_t(r) * a.N + j;
                uint32_t g = 0;
                for (; g + 4 <= gb; g += 4) {
                    uint32_t h[4][8];
                    pick_blocks<RULE, 4>(tabs, a.Bg, g, map, L, a.rows, h);
#pragma unroll
                    for (int q = 0; q < 4; ++q) store8_bits<OD>(a.out, ((b0 + g + q) * a.R + r) * a.N + j, h[q]);
                }
                for (; g < gb; ++g) {
                    uint32_t h[1][8];
                    pick_blocks<RULE, 1>(tabs, a.Bg, g, map, L, a.rows, h);
                    store8_bits<OD>(a.out, ((b0 + g) * a.R + r) * a.N + j, h[0]);
                }
            }
        } else {
            const uint32_t w = uint32_t(j1 - j0);
            for (uint32_t u = threadIdx.x; u < a.R * w; u += kDecThreads) {
                const uint32_t r = u / w;
                const int64_t j = j0 + (u % w);
                for (uint32_t g = 0; g < gb; ++g) {
                    uint32_t h = 0;
                    float m = 0.0f;
                    for (uint32_t rho = 0; rho < a.rows; ++rho) {
                        const uint32_t k = a.idx[int64_t(rho) * L + int64_t(r) * a.N + j];
                        const uint32_t v = tabs[g * a.Bg + (k < a.Bg ? k : 0)];
                        if (rho == 0) {
                            h = v;
                            m = __builtin_fabsf(f16_bits_to_f32(v));
                        } else {
                            keep<RULE>(h, m, v);
                        }
                    }
                    store1_bits<OD>(a.out, ((b0 + g) * a.R + r) * a.N + j, h);
                }
            }
        }
    } else if constexpr (VEC) {
        const uint32_t cpr = uint32_t((j1 - j0) / 8);   // 8-column chunks per row in the span
        for (uint32_t u = threadIdx.x; u < a.R * cpr; u += kDecThreads) {
            const uint32_t r = u / cpr;
            const int64_t j = j0 + int64_t(u % cpr) * 8;
            const u32x4 kv = *reinterpret_cast<const u32x4*>(a.idx + int64_t(r) * a.N + j);
            const uint32_t ks[8] = {kv.x & 0xFFFFu, kv.x >> 16, kv.y & 0xFFFFu, kv.y >> 16,
                                    kv.z & 0xFFFFu, kv.z >> 16, kv.w & 0xFFFFu, kv.w >> 16};
            uint32_t ka[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) ka[e] = ks[e] < a.Bg ? ks[e] : 0;
            uint32_t g = 0;
            for (; g + 4 <= gb; g += 4) {   // 32 gathers in flight, then 4 stores
                uint32_t h[4][8];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int e = 0; e < 8; ++e) h[q][e] = tabs[(g + q) * a.Bg + ka[e]];
#pragma unroll
                for (int q = 0; q < 4; ++q) store8_bits<OD>(a.out, ((b0 + g + q) * a.R + r) * a.N + j, h[q]);
            }
            for (; g < gb; ++g) {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = tabs[g * a.Bg + ka[e]];
                store8_bits<OD>(a.out, ((b0 + g) * a.R + r) * a.N + j, h);
            }
        }
    } else {
        const uint32_t w = uint32_t(j1 - j0);
        for (uint32_t u = threadIdx.x; u < a.R * w; u += kDecThreads) {
            const uint32_t r = u / w;
            const int64_t j = j0 + (u % w);
            const uint32_t k = a.idx[int64_t(r) * a.N + j];
            for (uint32_t g = 0; g < gb; ++g) {
                const uint32_t h = tabs[g * a.Bg + (k < a.Bg ? k : 0)];
                store1_bits<OD>(a.out, ((b0 + g) * a.R + r) * a.N + j, h);
            }
        }
    }
}

// Bucket of local index l in a table in memory, hashed per weight; with
// several rows, each row's bucket in its own segment and the pick.
template <bool MR, int RULE>
__device__ inline uint32_t hashed_bucket(const uint16_t* tab, uint32_t l, const DecArgs& a) {
    if constexpr (!MR) {
        return tab[bucket_of(l, a.seed, a.Bg)];
    } else {
        const uint32_t Bgr = a.Bg / a.rows;
        uint32_t h = tab[bucket_of(l, a.seed, Bgr)];
        float m = __builtin_fabsf(f16_bits_to_f32(h));
        for (uint32_t rho = 1; rho < a.rows; ++rho) keep<RULE>(h, m, tab[rho * Bgr + bucket_of(l, a.seed + rho, Bgr)]);
        return h;
    }
}

// One thread per 8 consecutive weights of a row (VEC) or per weight: hash
// the local index, read the bucket from the table in memory, write.
template <int OD, bool VEC, bool MR, int RULE>
__global__ __launch_bounds__(kDecThreads) void decode_hashed_kernel(DecArgs a) {
    const int64_t t = int64_t(blockIdx.x) * kDecThreads + threadIdx.x;
    if constexpr (VEC) {
        const int64_t cpr = a.N / 8;
        if (t >= a.M * cpr) return;
        const int64_t i = t / cpr, j = (t % cpr) * 8;
        const int64_t b = i / a.R;
        const uint32_t l0 = uint32_t((i % a.R) * a.N + j);
        uint32_t h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) h[e] = hashed_bucket<MR, RULE>(a.S + b * a.Bg, l0 + e, a);
        store8_bits<OD>(a.out, i * a.N + j, h);
    } else {
        if (t >= a.M * a.N) return;
        const int64_t i = t / a.N, j = t % a.N;
        const uint32_t l = uint32_t((i % a.R) * a.N + j);
        store1_bits<OD>(a.out, t, hashed_bucket<MR, RULE>(a.S + (i / a.R) * a.Bg, l, a));
    }
}

template <int OD, bool MR, int RULE>
void launch_map_v(const DecArgs& a, bool vec, unsigned grid, size_t lds, hipStream_t st) {
    if (vec)
        decode_map_kernel<OD, true, MR, RULE><<<grid, kDecThreads, lds, st>>>(a);
    else
        decode_map_kernel<OD, false, MR, RULE><<<grid, kDecThreads, lds, st>>>(a);
}

template <int OD>
sketch_status launch_map_typed(const DecArgs& a, int rule, bool vec, unsigned grid, size_t lds, hipStream_t st) {
    if (a.rows == 1)
        launch_map_v<OD, false, SKETCH_ABSMIN>(a, vec, grid, lds, st);
    else if (rule == SKETCH_ABSMIN)
        launch_map_v<OD, true, SKETCH_ABSMIN>(a, vec, grid, lds, st);
    else
        launch_map_v<OD, true, SKETCH_ABSMAX>(a, vec, grid, lds, st);
    return launch_status();
}

template <int OD, bool MR, int RULE>
void launch_hashed_v(const DecArgs& a, bool vec, unsigned grid, hipStream_t st) {
    if (vec)
        decode_hashed_kernel<OD, true, MR, RULE><<<grid, kDecThreads, 0, st>>>(a);
    else
        decode_hashed_kernel<OD, false, MR, RULE><<<grid, kDecThreads, 0, st>>>(a);
}

template <int OD>
sketch_status launch_hashed_typed(const DecArgs& a, int rule, bool vec, unsigned grid, hipStream_t st) {
    if (a.rows == 1)
        launch_hashed_v<OD, false, SKETCH_ABSMIN>(a, vec, grid, st);
    else if (rule == SKETCH_ABSMIN)
        launch_hashed_v<OD, true, SKETCH_ABSMIN>(a, vec, grid, st);
    else
        launch_hashed_v<OD, true, SKETCH_ABSMAX>(a, vec, grid, st);
    return launch_status();
}

int64_t decode_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu > 0 ? ncu : 256;
}

}  // namespace

sketch_status launch_decode(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                            void* out, sketch_dtype od, hipStream_t st) {
    const ProjLayout L = s.rows > 1 ? proj_layout_rows(s.R, s.N, s.rows) : proj_layout(s.R, s.N, s.Bg);
    DecArgs a;
    a.S = tables;
    a.idx = reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + L.idx);
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.out = out;
    a.M = s.M;
    a.N = s.N;
    a.nb = s.nb;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed = p->seed;
    a.rows = uint32_t(s.rows);
    // blocks per workgroup: as many tables as fit kDecTableLds (at least one)
    int64_t gb = int64_t(kDecTableLds / (size_t(s.Bg) * 2));
    gb = gb < 1 ? 1 : (gb > kDecMaxGroup ? kDecMaxGroup : gb);
    gb = gb < s.nb ? gb : s.nb;
    a.GB = uint32_t(gb);
    a.nbg = uint32_t((s.nb + gb - 1) / gb);
    // column spans: enough workgroups for four per CU, spans of >= 256 columns
    const bool vec = s.N % 8 == 0;
    const int64_t want = 4 * decode_cus();
    int64_t spans = (want + a.nbg - 1) / a.nbg;
    const int64_t max_spans = s.N / 256 > 0 ? s.N / 256 : 1;
    spans = spans < 1 ? 1 : (spans > max_spans ? max_spans : spans);
    int64_t span = (s.N + spans - 1) / spans;
    if (vec) span = (span + 7) / 8 * 8;
    spans = (s.N + span - 1) / span;
    a.span = uint32_t(span);
    const int64_t grid = int64_t(a.nbg) * spans;
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    const size_t lds = size_t(gb) * size_t(s.Bg) * 2;
    switch (od) {
        case SKETCH_F32: return launch_map_typed<SKETCH_F32>(a, p->rule, vec, unsigned(grid), lds, st);
        case SKETCH_BF16: return launch_map_typed<SKETCH_BF16>(a, p->rule, vec, unsigned(grid), lds, st);
        default: return launch_map_typed<SKETCH_F16>(a, p->rule, vec, unsigned(grid), lds, st);
    }
}

sketch_status launch_decode_hashed(const sketch_params* p, const Shape& s, const uint16_t* tables, void* out,
                                   sketch_dtype od, hipStream_t st) {
    DecArgs a = {};
    a.S = tables;
    a.out = out;
    a.M = s.M;
    a.N = s.N;
    a.nb = s.nb;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed = p->seed;
    a.rows = uint32_t(s.rows);
    const bool vec = s.N % 8 == 0;
    const int64_t threads = vec ? s.M * (s.N / 8) : s.M * s.N;
    const int64_t grid = (threads + kDecThreads - 1) / kDecThreads;
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    switch (od) {
        case SKETCH_F32: return launch_hashed_typed<SKETCH_F32>(a, p->rule, vec, unsigned(grid), st);
        case SKETCH_BF16: return launch_hashed_typed<SKETCH_BF16>(a, p->rule, vec, unsigned(grid), st);
        default: return launch_hashed_typed<SKETCH_F16>(a, p->rule, vec, unsigned(grid), st);
    }
}

}  // namespace sketch

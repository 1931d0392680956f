// encode.hip -- sketch compression on gfx950.
//
// "Resumen Técnico" › Metodología §1 (AbsMaxMin sketch): a bucket keeps the
// colliding weight of minimum absolute value.  Metodología §2: importance
// scales the choice (key = |w| * imp[j], one binary32 multiply).
// Metodología §4: selection and update are fused into one kernel, a MIN
// reduction through the projection P.
//
// Design (one workgroup per row block, persistent over blocks):
//   * The block's Bg buckets live in LDS as packed 64-bit words
//       word = key_bits << 32 | tie
//     where key_bits is the binary32 pattern of the non-negative key (its
//     unsigned order is the numeric order) and tie = l for AbsMin (LDS atomic
//     min: smaller key, then smaller l) or ~l for AbsMax (LDS atomic max:
//     larger key, then smaller l).  The result is independent of the order
//     in which lanes arrive, so the encode is deterministic.
//   * W is streamed once with 16-byte loads (8 bf16/fp16 or 2x4 fp32 per
//     chunk); the bucket of each position comes from the projection's
//     forward map (16-bit, shared by every block, cache-resident), so no hash
//     is recomputed per weight.
//   * After a barrier, each bucket's winner index is unpacked, the winning
//     weight is re-read (a cache hit: the block was just streamed) and
//     rounded to binary16; empty buckets store +0.
//   * Weight range (NaN/Inf, |w| >= 65520) and importance validity are
//     checked on the fly and reported through the status word.
#include "common.h"

namespace sketch {
namespace {

constexpr int kEncThreads = 512;
constexpr int kUnroll = 4;  // chunks in flight per thread

struct EncArgs {
    const void* W;
    const float* imp;
    const uint16_t* idx;
    const ProjHeader* hdr;
    uint16_t* S;
    int32_t* status;
    int64_t N, nb;
    uint32_t R, Bg, seed;
    uint32_t cpr;    // 8-element chunks per row (vector path)
    uint32_t nchunk; // chunks per block
};

template <int RULE>
__device__ inline void bucket_update(uint64_t* tab, uint32_t k, float key, uint32_t l) {
    uint64_t word = (uint64_t(__float_as_uint(key)) << 32) | uint64_t(RULE == SKETCH_ABSMIN ? l : ~l);
    if constexpr (RULE == SKETCH_ABSMIN)
        atomicMin(reinterpret_cast<unsigned long long*>(&tab[k]), (unsigned long long)word);
    else
        atomicMax(reinterpret_cast<unsigned long long*>(&tab[k]), (unsigned long long)word);
}

__device__ inline bool header_ok(const ProjHeader* h, const EncArgs& a) {
    return h->magic == kProjMagic && h->version == kProjVersion && h->R == a.R && h->N == uint32_t(a.N) &&
           h->Bg == a.Bg && h->seed == a.seed;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of one row, widened to float.  W is read once:
// non-temporal loads keep it from displacing the cached forward map.
template <int WDT>
__device__ inline void load8(const void* W, int64_t e0, float (&f)[8]) {
    if constexpr (WDT == SKETCH_F32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(W) + e0);
        f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + e0);
        u32x4 v = __builtin_nontemporal_load(p);
        uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (WDT == SKETCH_BF16) {
                f[2 * i] = __uint_as_float(u[i] << 16);
                f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
            } else {
                f[2 * i] = f16_bits_to_f32(u[i] & 0xFFFFu);
                f[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
            }
        }
    }
}

template <int WDT, int RULE, bool VEC>
__global__ __launch_bounds__(kEncThreads) void encode_kernel(EncArgs a) {
    extern __shared__ uint64_t tab[];
    const int tid = threadIdx.x;
    constexpr uint64_t kIdent = RULE == SKETCH_ABSMIN ? ~uint64_t(0) : uint64_t(0);

    if (!header_ok(a.hdr, a)) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(a.status, SKETCH_FLAG_PROJECTION);
        return;
    }

    const int64_t L = int64_t(a.R) * a.N;
    bool bad_w = false, bad_imp = false;

    for (int64_t b = blockIdx.x; b < a.nb; b += gridDim.x) {
        for (uint32_t q = tid; q < a.Bg; q += kEncThreads) tab[q] = kIdent;
        __syncthreads();

        const int64_t wbase = b * L;
        if constexpr (VEC) {
            // Thread walks chunks c = tid, tid + T, ...; (r, cc) tracked incrementally.
            const uint32_t dr = kEncThreads / a.cpr, dc = kEncThreads % a.cpr;
            uint32_t r = uint32_t(tid) / a.cpr, cc = uint32_t(tid) % a.cpr;
            for (uint32_t c0 = tid; c0 < a.nchunk; c0 += kEncThreads * kUnroll) {
                float w[kUnroll][8];
                uint4 kv[kUnroll];
                float im[kUnroll][8];
                uint32_t l0[kUnroll];
                bool live[kUnroll];
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    live[u] = c0 + uint32_t(u) * kEncThreads < a.nchunk;
                    l0[u] = r * uint32_t(a.N) + cc * 8;
                    if (live[u]) {
                        load8<WDT>(a.W, wbase + l0[u], w[u]);
                        kv[u] = *reinterpret_cast<const uint4*>(a.idx + l0[u]);
                        if (a.imp) {
                            const float4* ip = reinterpret_cast<const float4*>(a.imp + cc * 8);
                            float4 i0 = ip[0], i1 = ip[1];
                            im[u][0] = i0.x; im[u][1] = i0.y; im[u][2] = i0.z; im[u][3] = i0.w;
                            im[u][4] = i1.x; im[u][5] = i1.y; im[u][6] = i1.z; im[u][7] = i1.w;
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) im[u][e] = 1.0f;
                        }
                    }
                    cc += dc;
                    r += dr;
                    if (cc >= a.cpr) {
                        cc -= a.cpr;
                        ++r;
                    }
                }
#pragma unroll
                for (int u = 0; u < kUnroll; ++u) {
                    if (!live[u]) continue;
                    uint32_t ks[8] = {kv[u].x & 0xFFFFu, kv[u].x >> 16, kv[u].y & 0xFFFFu, kv[u].y >> 16,
                                      kv[u].z & 0xFFFFu, kv[u].z >> 16, kv[u].w & 0xFFFFu, kv[u].w >> 16};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float aw = __builtin_fabsf(w[u][e]);
                        bad_w |= !(aw < 65520.0f);
                        bad_imp |= !(im[u][e] >= 0.0f && im[u][e] <= 3.402823466e38f);
                        float key = aw * __builtin_fabsf(im[u][e]);
                        bucket_update<RULE>(tab, ks[e], key, l0[u] + e);
                    }
                }
            }
        } else {
            for (int64_t l = tid; l < L; l += kEncThreads) {
                const int64_t j = l % a.N;
                float f = load_elem<WDT>(a.W, wbase + l);
                float im = a.imp ? a.imp[j] : 1.0f;
                float aw = __builtin_fabsf(f);
                bad_w |= !(aw < 65520.0f);
                bad_imp |= !(im >= 0.0f && im <= 3.402823466e38f);
                bucket_update<RULE>(tab, a.idx[l], aw * __builtin_fabsf(im), uint32_t(l));
            }
        }
        __syncthreads();

        uint16_t* Sb = a.S + b * int64_t(a.Bg);
        for (uint32_t q = tid; q < a.Bg; q += kEncThreads) {
            uint64_t word = tab[q];
            uint16_t v = 0;
            if (word != kIdent) {
                uint32_t l = uint32_t(word);
                if constexpr (RULE == SKETCH_ABSMAX) l = ~l;
                v = f32_to_f16_bits(load_elem<WDT>(a.W, wbase + l));
            }
            Sb[q] = v;
        }
        __syncthreads();
    }
    int32_t flags = (bad_w ? SKETCH_FLAG_WEIGHT_RANGE : 0) | (bad_imp ? SKETCH_FLAG_IMPORTANCE : 0);
    if (flags) atomicOr(a.status, flags);
}

template <int WDT, int RULE>
sketch_status launch_typed(const EncArgs& a, bool vec, hipStream_t st) {
    const size_t lds = size_t(a.Bg) * sizeof(uint64_t);
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    int64_t grid = a.nb < int64_t(ncu) * 4 ? a.nb : int64_t(ncu) * 4;
    if (vec)
        encode_kernel<WDT, RULE, true><<<unsigned(grid), kEncThreads, lds, st>>>(a);
    else
        encode_kernel<WDT, RULE, false><<<unsigned(grid), kEncThreads, lds, st>>>(a);
    return launch_status();
}

}  // namespace

sketch_status launch_encode(const sketch_params* p, const Shape& s, const void* proj, const void* W,
                            const float* imp, uint16_t* tables, int32_t* status, hipStream_t st) {
    if (s.nb == 0) return SKETCH_OK;
    const ProjLayout L = proj_layout(s.R, s.N, s.Bg);
    EncArgs a;
    a.W = W;
    a.imp = imp;
    a.idx = reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + L.idx);
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.S = tables;
    a.status = status;
    a.N = s.N;
    a.nb = s.nb;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed = p->seed;
    a.cpr = uint32_t(s.N / 8);
    a.nchunk = uint32_t(s.R * s.N / 8);
    // Vector path: rows are whole 8-element chunks (16-byte aligned given a
    // 16-byte aligned W) and the importance vector is 16-byte aligned.
    const bool vec = (s.N % 8 == 0) && (reinterpret_cast<uintptr_t>(imp) % 16 == 0);
    const int rule = p->rule;
    switch (p->w_dtype) {
        case SKETCH_F32:
            return rule == SKETCH_ABSMIN ? launch_typed<SKETCH_F32, SKETCH_ABSMIN>(a, vec, st)
                                         : launch_typed<SKETCH_F32, SKETCH_ABSMAX>(a, vec, st);
        case SKETCH_BF16:
            return rule == SKETCH_ABSMIN ? launch_typed<SKETCH_BF16, SKETCH_ABSMIN>(a, vec, st)
                                         : launch_typed<SKETCH_BF16, SKETCH_ABSMAX>(a, vec, st);
        case SKETCH_F16:
            return rule == SKETCH_ABSMIN ? launch_typed<SKETCH_F16, SKETCH_ABSMIN>(a, vec, st)
                                         : launch_typed<SKETCH_F16, SKETCH_ABSMAX>(a, vec, st);
    }
    return SKETCH_EINVAL;
}

}  // namespace sketch

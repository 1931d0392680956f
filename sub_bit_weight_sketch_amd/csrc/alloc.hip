// alloc.hip -- importance-aware space allocation.
//
// "Resumen Técnico" › Metodología §2: rows of higher importance (expected
// squared activation E[a^2]) receive more sketch space.  Readings (the pages
// give no formulas): the unit is the row block; its importance is
// s_b = sum_{i in b} sum_j W[i][j]^2 E[x_j^2] (sketch_block_importance);
// the counts Bg_b keep the uniform budget and are shared by largest
// remainder (sketch_alloc_plan, host); block b hashes with the same function
// reduced to its own count, k_b(l) = umulhi(H[l], Bg_b) with
// H[l] = fmix32((l * 0x9E3779B1) ^ seed), and owns tables[off[b] ..).
//
// The projection of an allocated sketch is H itself (uint32 per local index,
// shared by every block).  W_hat no longer factors through one P for all
// blocks, so the products decode every weight (one 16-byte slice of H per 4
// columns, one multiply-high and one LDS gather per weight).  A block whose
// offsets are out of range (count 0 or above bg_max, or past the uniform
// budget) gives NaN rows; a projection of another kind or shape gives NaN.
#include "common.h"
#include "dgemm.h"

namespace sketch {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAThreads = 256;
constexpr int kAMaxTok = 16;   // tokens per GEMV pass

__device__ inline bool hash_header_ok(const ProjHeader* h, uint32_t R, int64_t N, uint32_t seed) {
    return h->magic == kProjMagicHash && h->version == kProjVersion && h->R == R && h->N == uint32_t(N) &&
           h->seed == seed;
}

// ------------------------------------------------------------- projection
// (the header is cleared here and written by a launch after this one)
__global__ void alloc_proj_kernel(ProjHeader* hdr, uint32_t* H, int64_t L, uint32_t seed) {
    const int64_t l = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (l == 0) *hdr = ProjHeader{0, 0, 0, 0, 0, 0, {0, 0}};
    if (l < L) H[l] = fmix32((uint32_t(l) * 0x9E3779B1u) ^ seed);
}

// -------------------------------------------------------- block importance
// One workgroup per row block: each thread sums w^2 * a2[j] over a fixed set
// of the block's elements (8 columns at a time when N % 8 == 0), then a
// fixed binary tree in LDS adds the 256 partial sums: the same float32
// order on every run.
template <int WDT, bool VEC>
__global__ __launch_bounds__(kAThreads) void block_importance_kernel(const void* W, const float* a2, float* scores,
                                                                     int64_t N, int64_t nb, uint32_t R) {
    __shared__ float red[kAThreads];
    const int64_t L = int64_t(R) * N;
    for (int64_t b = blockIdx.x; b < nb; b += gridDim.x) {
        float acc = 0.0f;
        if constexpr (VEC) {
            // four 8-element chunks per thread in flight (their loads first)
            constexpr int U = 4;
            for (int64_t base = int64_t(threadIdx.x) * 8; base < L; base += int64_t(U) * kAThreads * 8) {
                float w[U][8];
                int64_t jj[U];
                bool in[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int64_t l0 = base + int64_t(u) * kAThreads * 8;
                    in[u] = l0 < L;
                    const int64_t lc = in[u] ? l0 : 0;   // clamped: an unused chunk re-reads the first
                    jj[u] = lc % N;
                    if constexpr (WDT == SKETCH_F32) {
                        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const float*>(W) + b * L + lc);
                        const u32x4 x = __builtin_nontemporal_load(p), y = __builtin_nontemporal_load(p + 1);
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            w[u][e] = __uint_as_float(x[e]);
                            w[u][4 + e] = __uint_as_float(y[e]);
                        }
                    } else {
                        const u32x4 v = __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + b * L + lc));
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const uint32_t h = (v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
                            w[u][e] = WDT == SKETCH_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
                        }
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (!in[u]) continue;
                    const float4 x0 = *reinterpret_cast<const float4*>(a2 + jj[u]);
                    const float4 x1 = *reinterpret_cast<const float4*>(a2 + jj[u] + 4);
                    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += w[u][e] * w[u][e] * xs[e];
                }
            }
        } else {
            for (int64_t l = threadIdx.x; l < L; l += kAThreads) {
                const float w = load_elem<WDT>(W, b * L + l);
                acc += w * w * a2[l % N];
            }
        }
        red[threadIdx.x] = acc;
        __syncthreads();
        for (int s = kAThreads / 2; s > 0; s >>= 1) {
            if (int(threadIdx.x) < s) red[threadIdx.x] += red[threadIdx.x + s];
            __syncthreads();
        }
        if (threadIdx.x == 0) scores[b] = red[0];
        __syncthreads();
    }
}

// ------------------------------------------------------------------ GEMV
struct AllocArgs {
    const uint16_t* S;
    const uint32_t* H;       // hash of every local index (projection)
    const ProjHeader* hdr;
    const uint32_t* boff;
    const void* X;
    float* Y;
    int64_t T, M, N, nb, t0;
    uint64_t total;          // uniform budget nb * Bg
    uint32_t R, seed, bg_max, ntok;
};

constexpr uint32_t kARowsPerWg = kAThreads / 64;
constexpr int kAAhead = 4;   // 8-column chunks per lane whose loads go out together

// One wave per weight row: a workgroup takes 4 rows of one block and stages
// the block's Bg_b buckets in LDS.  Lane c walks the 8-column chunks c,
// c + 64, ...: two 16-byte slices of H, 8 multiply-highs and 8 LDS gathers
// give the 8 weights, which multiply x[t][j .. j+7] into the token's partial
// sum; a fixed xor butterfly adds the 64 partial sums (deterministic).
template <int XDT, bool VEC>
__global__ __launch_bounds__(kAThreads) void alloc_gemv_kernel(AllocArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t tab[];   // [bg_max]
    const uint32_t rgroups = (a.R + kARowsPerWg - 1) / kARowsPerWg;
    const int64_t b = blockIdx.x / rgroups;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t r = (blockIdx.x % rgroups) * kARowsPerWg + (threadIdx.x >> 6);
    uint32_t off0 = 0, bgb = 1;
    const bool ok = hash_header_ok(a.hdr, a.R, a.N, a.seed) && alloc_block(a.boff, b, a.bg_max, a.total, off0, bgb);
    if (ok)
        for (uint32_t q = threadIdx.x; q < bgb; q += kAThreads) tab[q] = a.S[off0 + q];
    __syncthreads();
    if (r >= a.R) return;   // whole waves; no barrier follows
    float acc[kAMaxTok];
#pragma unroll
    for (int t = 0; t < kAMaxTok; ++t) acc[t] = 0.0f;
    if (ok) {
        const uint32_t* Hr = a.H + int64_t(r) * a.N;
        if constexpr (VEC) {
            // kAAhead chunks per round: their hash slices and the first
            // token's x go out together (unconditional loads; chunks past the
            // row re-read the round's first one and are skipped)
            for (int64_t j0 = int64_t(lane) * 8; j0 < a.N; j0 += kAAhead * 64 * 8) {
                u32x4 hv[kAAhead][2];
                float x0[kAAhead][8];
#pragma unroll
                for (int u = 0; u < kAAhead; ++u) {
                    const int64_t j = j0 + u * 64 * 8 < a.N ? j0 + u * 64 * 8 : j0;
                    hv[u][0] = *reinterpret_cast<const u32x4*>(Hr + j);
                    hv[u][1] = *reinterpret_cast<const u32x4*>(Hr + j + 4);
                    load8_f32<XDT>(a.X, a.t0 * a.N + j, x0[u]);
                }
#pragma unroll
                for (int u = 0; u < kAAhead; ++u) {
                    const int64_t j = j0 + u * 64 * 8;
                    if (j < a.N) {
                        float w[8];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            w[e] = f16_bits_to_f32(tab[__umulhi(hv[u][0][e], bgb)]);
                            w[4 + e] = f16_bits_to_f32(tab[__umulhi(hv[u][1][e], bgb)]);
                        }
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[0] += w[e] * x0[u][e];
#pragma unroll
                        for (int t = 1; t < kAMaxTok; ++t)
                            if (uint32_t(t) < a.ntok) {
                                float xv[8];
                                load8_f32<XDT>(a.X, (a.t0 + t) * a.N + j, xv);
#pragma unroll
                                for (int e = 0; e < 8; ++e) acc[t] += w[e] * xv[e];
                            }
                    }
                }
            }
        } else {
            for (int64_t j = lane; j < a.N; j += 64) {
                const float w = f16_bits_to_f32(tab[__umulhi(Hr[j], bgb)]);
#pragma unroll
                for (int t = 0; t < kAMaxTok; ++t)
                    if (uint32_t(t) < a.ntok) acc[t] += w * load_elem<XDT>(a.X, (a.t0 + t) * a.N + j);
            }
        }
    }
    float mine = 0.0f;   // lane t keeps token t's sum
#pragma unroll
    for (int t = 0; t < kAMaxTok; ++t) {
        if (uint32_t(t) >= a.ntok) break;
        float v = acc[t];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == uint32_t(t)) mine = v;
    }
    if (lane < a.ntok) a.Y[(a.t0 + lane) * a.M + b * a.R + r] = ok ? mine : __builtin_nanf("");
}

// ------------------------------------------------------------------ GEMM
// The decoded-W_hat skeleton (dgemm.h): 256 tokens x 128 outputs per
// workgroup.  Each of the tile's row blocks has its own LDS slot of bg_max
// buckets staged from its own offset, so a block's validity does not depend
// on its neighbours.
constexpr int kGTM = 256, kGTN = dgemm::kTN;

inline int64_t alloc_tile_blocks(int64_t R, int64_t nb) {
    const int64_t n = (kGTN - 1) / R + 2;
    return n < nb ? n : nb;
}

inline size_t alloc_gemm_lds(const Shape& s) {
    return size_t(dgemm::kWBytes) + size_t(2 * s.R * 8 * 16) +
           size_t(alloc_tile_blocks(s.R, s.nb)) * size_t(s.bg_max) * 2;
}

// Decode policy: per chunk the hashes of the R rows' positions (R x 8
// pieces of 4 columns, 32-bit); a weight's bucket is the multiply-high of
// its hash by its block's count, read from the block's LDS slot; a thread
// decodes 16 columns of one output row.  Rows of an invalid block decode to
// NaN.
struct AllocDecode {
    typedef AllocArgs Args;
    static constexpr int kThreads = 256, kSchedLds = 2, kSchedValu = 8;
    static constexpr bool kScaled = false;
    const Args& a;
    const int tid, jseg;
    const uint32_t hslices;   // 16-byte hash slices per chunk (<= 256)
    uint32_t* Hs;             // [2][R][kBK]
    uint16_t* Ss;             // [slots][bg_max]
    int64_t bA, bB;
    uint32_t mpc;
    int64_t moff;
    bool orow_ok, bad;
    uint32_t r_d, bgb;
    const uint16_t* Sblk;

    __device__ AllocDecode(const Args& args, unsigned char* region, int tid_, int64_t o0, int o_d, int jseg_)
        : a(args), tid(tid_), jseg(jseg_), hslices(args.R * 8) {
        Hs = reinterpret_cast<uint32_t*>(region);
        Ss = reinterpret_cast<uint16_t*>(Hs + 2 * hslices * 4);
        bA = o0 / a.R;
        bB = (o0 + dgemm::kTN - 1) / a.R;
        if (bB > a.nb - 1) bB = a.nb - 1;
        // slice q = (r, piece), one per thread at most, loaded from a clamped
        // address (a clamped slice is never used: columns past N decode to 0)
        const uint32_t mq = uint32_t(tid) < hslices ? uint32_t(tid) : hslices - 1;
        mpc = (mq & 7) * 4;
        moff = int64_t(mq >> 3) * a.N + mpc;
        const int64_t orow = o0 + o_d;
        orow_ok = orow < a.M;
        r_d = orow_ok ? uint32_t(orow % a.R) : 0;
        const int64_t ob = orow_ok ? orow / a.R : bA;
        uint32_t boff0 = 0;
        bgb = 1;
        bad = orow_ok && !alloc_block(a.boff, ob, a.bg_max, a.total, boff0, bgb);
        if (bad) bgb = 1;   // keep the gathers inside the slot
        Sblk = Ss + (ob - bA) * a.bg_max;
    }
    __device__ bool header_ok() const { return hash_header_ok(a.hdr, a.R, a.N, a.seed); }
    __device__ void stage() const {   // tables of blocks bA .. bB, one slot of bg_max buckets each
        for (int64_t b = bA; b <= bB; ++b) {
            uint32_t off, cnt;
            if (alloc_block(a.boff, b, a.bg_max, a.total, off, cnt))
                for (uint32_t q = tid; q < cnt; q += kThreads) Ss[(b - bA) * a.bg_max + q] = a.S[off + q];
        }
    }
    __device__ void map_load(int64_t j0, dgemm::u32x4& mv) const {
        const bool in = j0 + mpc < a.N;
        mv = *reinterpret_cast<const dgemm::u32x4*>(a.H + (in ? moff + j0 : moff - mpc + a.N - 4));
    }
    __device__ void map_store(int buf, const dgemm::u32x4& mv) const {
        if (uint32_t(tid) < hslices) *reinterpret_cast<dgemm::u32x4*>(Hs + (buf * hslices + tid) * 4) = mv;
    }
    // Straight-line (in-bounds data whatever the row and column, then a
    // select), so the decode shares one basic block with the MFMAs it is
    // interleaved with.
    __device__ void decode(int buf, int64_t j0, uint16_t* dst) const {
        const uint32_t* hb = Hs + buf * hslices * 4 + r_d * dgemm::kBK + jseg;
        uint32_t pk[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const dgemm::u32x4 h0 = *reinterpret_cast<const dgemm::u32x4*>(hb + hh * 8);
            const dgemm::u32x4 h1 = *reinterpret_cast<const dgemm::u32x4*>(hb + hh * 8 + 4);
            uint32_t v[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = Sblk[__umulhi(h0[e], bgb)];
                v[4 + e] = Sblk[__umulhi(h1[e], bgb)];
            }
            const bool use = orow_ok && j0 + jseg + hh * 8 < a.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w = (__float_as_uint(f16_bits_to_f32(v[2 * e])) >> 16) |
                                   (__float_as_uint(f16_bits_to_f32(v[2 * e + 1])) & 0xFFFF0000u);
                pk[hh * 4 + e] = !use ? 0u : (bad ? 0x7FC07FC0u : w);
            }
        }
        dgemm::u32x4* d = reinterpret_cast<dgemm::u32x4*>(dst);
        d[0] = dgemm::u32x4{pk[0], pk[1], pk[2], pk[3]};
        d[1] = dgemm::u32x4{pk[4], pk[5], pk[6], pk[7]};
    }
    __device__ float out_scale(int64_t) const { return 1.0f; }
};

// ---------------------------------------------------------------- decode
struct ADecArgs {
    const uint16_t* S;
    const uint32_t* H;       // projection hashes (map form only)
    const ProjHeader* hdr;   // (map form only)
    const uint32_t* boff;
    void* out;
    int64_t N, nb;
    uint64_t total;
    uint32_t R, seed, bg_max, spans, span;
};

// One workgroup per (row block, column span).  Map form: the block's table
// is staged in LDS and each bucket index comes from the projection's hash
// slices; HASHED: every weight's hash is computed and its bucket read from
// the table in memory (the naive baseline).  Invalid blocks and a
// projection of another kind or shape give NaN.
template <int OD, bool VEC, bool HASHED>
__global__ __launch_bounds__(kAThreads) void alloc_decode_kernel(ADecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t tab[];   // [bg_max] (map form)
    const int64_t b = blockIdx.x / a.spans;
    const int64_t j0 = int64_t(blockIdx.x % a.spans) * a.span;
    const int64_t j1 = j0 + a.span < a.N ? j0 + a.span : a.N;
    uint32_t off0 = 0, bgb = 1;
    bool ok = alloc_block(a.boff, b, a.bg_max, a.total, off0, bgb);
    if constexpr (!HASHED) {
        ok = ok && hash_header_ok(a.hdr, a.R, a.N, a.seed);
        if (ok)
            for (uint32_t q = threadIdx.x; q < bgb; q += kAThreads) tab[q] = a.S[off0 + q];
        __syncthreads();
    }
    const uint16_t* Sb = a.S + off0;
    constexpr uint32_t kNaN16 = 0x7E00u;
    if constexpr (VEC) {
        const uint32_t cpr = uint32_t((j1 - j0) / 8);
        for (uint32_t u = threadIdx.x; u < a.R * cpr; u += kAThreads) {
            const uint32_t r = u / cpr;
            const int64_t j = j0 + int64_t(u % cpr) * 8;
            const int64_t e0 = (b * a.R + r) * a.N + j;
            uint32_t h[8];
            if (!ok) {
#pragma unroll
                for (int e = 0; e < 8; ++e) h[e] = kNaN16;
            } else if constexpr (HASHED) {
                const uint32_t l0 = uint32_t(r * a.N + j);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    h[e] = Sb[__umulhi(fmix32(((l0 + e) * 0x9E3779B1u) ^ a.seed), bgb)];
            } else {
                const uint32_t* hp = a.H + int64_t(r) * a.N + j;
                const u32x4 h0 = *reinterpret_cast<const u32x4*>(hp);
                const u32x4 h1 = *reinterpret_cast<const u32x4*>(hp + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = tab[__umulhi(h0[e], bgb)];
                    h[4 + e] = tab[__umulhi(h1[e], bgb)];
                }
            }
            store8_bits<OD>(a.out, e0, h);
        }
    } else {
        const uint32_t w = uint32_t(j1 - j0);
        for (uint32_t u = threadIdx.x; u < a.R * w; u += kAThreads) {
            const uint32_t r = u / w;
            const int64_t j = j0 + (u % w);
            uint32_t h = kNaN16;
            if (ok) {
                const uint32_t l = uint32_t(r * a.N + j);
                if constexpr (HASHED)
                    h = Sb[__umulhi(fmix32((l * 0x9E3779B1u) ^ a.seed), bgb)];
                else
                    h = tab[__umulhi(a.H[l], bgb)];
            }
            store1_bits<OD>(a.out, (b * a.R + r) * a.N + j, h);
        }
    }
}

inline int64_t alloc_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu > 0 ? ncu : 256;
}

template <int OD, bool HASHED>
void launch_adec(const ADecArgs& a, bool vec, unsigned grid, size_t lds, hipStream_t st) {
    if (vec)
        alloc_decode_kernel<OD, true, HASHED><<<grid, kAThreads, lds, st>>>(a);
    else
        alloc_decode_kernel<OD, false, HASHED><<<grid, kAThreads, lds, st>>>(a);
}

}  // namespace

sketch_status launch_projection_build_hash(const sketch_params* p, const Shape& s, void* proj, hipStream_t st) {
    const ProjLayout L = proj_layout_hash(s.R, s.N);
    char* base = static_cast<char*>(proj);
    ProjHeader h{kProjMagicHash, kProjVersion, uint32_t(s.R), uint32_t(s.N), uint32_t(s.Bg), p->seed, {0, 0}};
    const int64_t n = s.R * s.N;
    alloc_proj_kernel<<<unsigned((n + 255) / 256), 256, 0, st>>>(reinterpret_cast<ProjHeader*>(base),
                                                                reinterpret_cast<uint32_t*>(base + L.idx), n, p->seed);
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    return launch_proj_header(proj, h, st);
}

sketch_status launch_block_importance(const sketch_params* p, const Shape& s, const void* W, const float* a2,
                                      float* scores, hipStream_t st) {
    const int64_t cap = 4 * alloc_cus();
    const unsigned grid = unsigned(s.nb < cap ? s.nb : cap);
    const bool vec = s.N % 8 == 0 && (reinterpret_cast<uintptr_t>(a2) & 15) == 0;
#define SKETCH_BI(WDT)                                                                                     \
    (vec ? (block_importance_kernel<WDT, true><<<grid, kAThreads, 0, st>>>(W, a2, scores, s.N, s.nb, uint32_t(s.R)), 0) \
         : (block_importance_kernel<WDT, false><<<grid, kAThreads, 0, st>>>(W, a2, scores, s.N, s.nb, uint32_t(s.R)), 0))
    switch (p->w_dtype) {
        case SKETCH_F32: SKETCH_BI(SKETCH_F32); break;
        case SKETCH_BF16: SKETCH_BI(SKETCH_BF16); break;
        default: SKETCH_BI(SKETCH_F16); break;
    }
#undef SKETCH_BI
    return launch_status();
}

bool gemm_alloc_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch) {
    return p->w_dtype == SKETCH_BF16 && xdt == SKETCH_BF16 && batch > kAMaxTok && s.N % 8 == 0 && s.R * 8 <= 256 &&
           alloc_gemm_lds(s) <= 160 * 1024;
}

sketch_status launch_matmul_alloc(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                                  const void* X, sketch_dtype xdt, int64_t batch, float* Y, hipStream_t st) {
    AllocArgs a;
    a.S = tables;
    a.H = reinterpret_cast<const uint32_t*>(static_cast<const char*>(proj) + proj_layout_hash(s.R, s.N).idx);
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.boff = s.boff;
    a.X = X;
    a.Y = Y;
    a.T = batch;
    a.M = s.M;
    a.N = s.N;
    a.nb = s.nb;
    a.t0 = 0;
    a.total = uint64_t(s.nb) * uint64_t(s.Bg);
    a.R = uint32_t(s.R);
    a.seed = p->seed;
    a.bg_max = uint32_t(s.bg_max);
    a.ntok = 0;
    if (gemm_alloc_supported(p, s, xdt, batch)) {
        static_assert(kGTM == AllocDecode::kThreads, "the kernel numbers its tiles with this token tile");
        const uint32_t tiles_m = uint32_t((s.M + kGTN - 1) / kGTN);
        const int64_t grid = int64_t(tiles_m) * ((batch + kGTM - 1) / kGTM);
        if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
        dgemm::dgemm_kernel<AllocDecode><<<unsigned(grid), AllocDecode::kThreads, alloc_gemm_lds(s), st>>>(a, tiles_m, 1u,
                                                                                                      nullptr);
        return launch_status();
    }
    const bool vec = s.N % 8 == 0;
    const int64_t grid = s.nb * ((s.R + kARowsPerWg - 1) / kARowsPerWg);
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    const size_t lds = size_t(s.bg_max) * 2;
    for (int64_t t0 = 0; t0 < batch; t0 += kAMaxTok) {
        a.t0 = t0;
        a.ntok = uint32_t(batch - t0 < kAMaxTok ? batch - t0 : kAMaxTok);
#define SKETCH_AGEMV(XDT)                                                                                 \
    (vec ? (alloc_gemv_kernel<XDT, true><<<unsigned(grid), kAThreads, lds, st>>>(a), 0)                  \
         : (alloc_gemv_kernel<XDT, false><<<unsigned(grid), kAThreads, lds, st>>>(a), 0))
        switch (xdt) {
            case SKETCH_F32: SKETCH_AGEMV(SKETCH_F32); break;
            case SKETCH_BF16: SKETCH_AGEMV(SKETCH_BF16); break;
            default: SKETCH_AGEMV(SKETCH_F16); break;
        }
#undef SKETCH_AGEMV
        if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    }
    return SKETCH_OK;
}

sketch_status launch_decode_alloc(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                                  void* out, sketch_dtype od, bool hashed, hipStream_t st) {
    ADecArgs a;
    a.S = tables;
    a.H = proj ? reinterpret_cast<const uint32_t*>(static_cast<const char*>(proj) + proj_layout_hash(s.R, s.N).idx)
               : nullptr;
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.boff = s.boff;
    a.out = out;
    a.N = s.N;
    a.nb = s.nb;
    a.total = uint64_t(s.nb) * uint64_t(s.Bg);
    a.R = uint32_t(s.R);
    a.seed = p->seed;
    a.bg_max = uint32_t(s.bg_max);
    // column spans: enough workgroups for four per CU, spans of >= 256 columns
    const bool vec = s.N % 8 == 0;
    const int64_t want = 4 * alloc_cus();
    int64_t spans = (want + s.nb - 1) / s.nb;
    const int64_t max_spans = s.N / 256 > 0 ? s.N / 256 : 1;
    spans = spans < 1 ? 1 : (spans > max_spans ? max_spans : spans);
    int64_t span = (s.N + spans - 1) / spans;
    if (vec) span = (span + 7) / 8 * 8;
    spans = (s.N + span - 1) / span;
    a.spans = uint32_t(spans);
    a.span = uint32_t(span);
    const int64_t grid = s.nb * spans;
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    const size_t lds = hashed ? 0 : size_t(s.bg_max) * 2;
    switch (od) {
        case SKETCH_F32:
            hashed ? launch_adec<SKETCH_F32, true>(a, vec, unsigned(grid), lds, st)
                   : launch_adec<SKETCH_F32, false>(a, vec, unsigned(grid), lds, st);
            break;
        case SKETCH_BF16:
            hashed ? launch_adec<SKETCH_BF16, true>(a, vec, unsigned(grid), lds, st)
                   : launch_adec<SKETCH_BF16, false>(a, vec, unsigned(grid), lds, st);
            break;
        default:
            hashed ? launch_adec<SKETCH_F16, true>(a, vec, unsigned(grid), lds, st)
                   : launch_adec<SKETCH_F16, false>(a, vec, unsigned(grid), lds, st);
            break;
    }
    return launch_status();
}

}  // namespace sketch

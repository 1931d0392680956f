// rows.hip -- the multi-row AbsMaxMin sketch.
//
// "Resumen Técnico" › Metodología §1 (multi-row design): several independent
// hash functions, each with its own sketch row, so that weights of similar
// value are more likely to share a bucket in some row; decompression takes
// the Max over the rows.  Readings (the pages give no formulas for them):
//   * row rho (0 <= rho < rows) hashes with seed + rho;
//   * the block's Bg buckets are split into `rows` contiguous segments of
//     Bgr = Bg / rows (same bits per weight, same [nb][Bg] table layout); row
//     rho's bucket of local index l is rho * Bgr + k_rho(l), k_rho taken over
//     Bgr buckets;
//   * every row keeps, per bucket, the same winner as the single-row sketch
//     (AbsMin: smallest key |w| * imp[j], then smallest l);
//   * W_hat[i][j] is the row bucket of largest magnitude (AbsMin; smallest
//     for AbsMax), the first row among equal magnitudes.
// W_hat is no longer linear in the tables, so the product cannot factor
// through Z = P^T x: every kernel here decodes each weight it uses.
//
// Projection of a multi-row sketch: the header (magic kProjMagicRows, the row
// count in pad[0]) and the forward maps of all rows, idx[rho][l] (indices
// into the block's Bg).  Single-row kernels reject it by its magic.
#include "common.h"

namespace sketch {
namespace {

constexpr int kRowsThreads = 256;
constexpr int kRowsMaxTok = 16;   // tokens per GEMV pass

__device__ inline bool rows_header_ok(const ProjHeader* h, uint32_t R, int64_t N, uint32_t Bg, uint32_t seed,
                                      uint32_t rows) {
    return h->magic == kProjMagicRows && h->version == kProjVersion && h->R == R && h->N == uint32_t(N) &&
           h->Bg == Bg && h->seed == seed && h->pad[0] == rows;
}

// Bucket of position l whose row candidates are (b0 + idx[rho * L + l]):
// the one of largest magnitude (AbsMin) or smallest (AbsMax), first row on
// ties.  NaN never replaces an earlier candidate.
template <int RULE>
__device__ inline uint32_t pick(const uint16_t* tab, const uint16_t* idx, int64_t L, int64_t l, uint32_t rows) {
    uint32_t best = tab[idx[l]];
    float bm = __builtin_fabsf(f16_bits_to_f32(best));
    for (uint32_t rho = 1; rho < rows; ++rho) {
        const uint32_t v = tab[idx[int64_t(rho) * L + l]];
        const float m = __builtin_fabsf(f16_bits_to_f32(v));
        if (RULE == SKETCH_ABSMIN ? m > bm : m < bm) {
            best = v;
            bm = m;
        }
    }
    return best;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The picks of 8 consecutive positions l0 .. l0+7 whose row indices are the
// 16-byte slices idx[rho * L + l0 ..]: bucket bits in h.
template <int RULE>
__device__ inline void pick8(const uint16_t* tab, const uint16_t* idx, int64_t L, int64_t l0, uint32_t rows,
                             uint32_t (&h)[8]) {
    float bm[8];
    {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(idx + l0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h[e] = tab[(kv[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu];
            bm[e] = __builtin_fabsf(f16_bits_to_f32(h[e]));
        }
    }
    for (uint32_t rho = 1; rho < rows; ++rho) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(idx + int64_t(rho) * L + l0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t v = tab[(kv[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu];
            const float m = __builtin_fabsf(f16_bits_to_f32(v));
            if (RULE == SKETCH_ABSMIN ? m > bm[e] : m < bm[e]) {
                h[e] = v;
                bm[e] = m;
            }
        }
    }
}

// -------------------------------------------------------------- projection
__global__ void rows_proj_kernel(ProjHeader* hdr, ProjHeader h, uint16_t* idx, int64_t L, uint32_t rows,
                                 uint32_t Bgr, uint32_t seed) {
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e == 0) *hdr = h;
    if (e >= L * rows) return;
    const uint32_t rho = uint32_t(e / L);
    const uint32_t l = uint32_t(e % L);
    idx[e] = uint16_t(rho * Bgr + bucket_of(l, seed + rho, Bgr));
}

// ------------------------------------------------------------- GEMV (batch)
struct RowsGemvArgs {
    const uint16_t* S;
    const uint16_t* idx;
    const ProjHeader* hdr;
    const void* X;
    float* Y;
    int64_t M, N, nb, t0;
    uint32_t R, Bg, seed, rows, ntok;
    uint32_t tpr;   // threads per weight row (kRowsThreads / rows handled together)
};

// x[t][j0 .. j0+7] widened to float (16- or 32-byte aligned loads).
template <int XDT>
__device__ inline void load_x8(const void* X, int64_t e0, float (&f)[8]) {
    if constexpr (XDT == SKETCH_F32) {
        const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(X) + e0);
        const float4 u = p[0], v = p[1];
        f[0] = u.x; f[1] = u.y; f[2] = u.z; f[3] = u.w; f[4] = v.x; f[5] = v.y; f[6] = v.z; f[7] = v.w;
    } else {
        const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(X) + e0);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h = (v[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
            f[e] = XDT == SKETCH_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
        }
    }
}

// One workgroup per row block (persistent over blocks).  The block's table
// sits in LDS; thread (r, c) of a pass walks the 8-column chunks c, c + tpr,
// ... of weight row r: one 16-byte slice of each sketch row's forward map,
// 8 gathers per sketch row from LDS and the pick give 8 decoded weights,
// which multiply x[t][j .. j+7] (one 16-byte load per token) into the
// token's partial sum.  The tpr partial sums of a row are added in LDS in
// thread order (deterministic).  VEC: N % 8 == 0; otherwise one weight at a
// time.
template <int XDT, int RULE, bool VEC>
__global__ __launch_bounds__(kRowsThreads) void rows_gemv_kernel(RowsGemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    uint16_t* tab = reinterpret_cast<uint16_t*>(lds);                                        // [Bg]
    float* red = reinterpret_cast<float*>(lds + ((size_t(a.Bg) * 2 + 15) & ~size_t(15)));    // [ntok][256]
    const bool ok = rows_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed, a.rows);
    const int64_t L = int64_t(a.R) * a.N;
    const uint32_t rpp = kRowsThreads / a.tpr;   // weight rows per pass over the block
    const uint32_t c = threadIdx.x % a.tpr, rr = threadIdx.x / a.tpr;
    for (int64_t b = blockIdx.x; b < a.nb; b += gridDim.x) {
        for (uint32_t q = threadIdx.x; q < a.Bg; q += kRowsThreads) tab[q] = a.S[b * a.Bg + q];
        __syncthreads();
        for (uint32_t r0 = 0; r0 < a.R; r0 += rpp) {
            const uint32_t r = r0 + rr;
            float acc[kRowsMaxTok];
#pragma unroll
            for (int t = 0; t < kRowsMaxTok; ++t) acc[t] = 0.0f;
            if (rr < rpp && r < a.R && ok) {
                if constexpr (VEC) {
                    for (int64_t j = int64_t(c) * 8; j < a.N; j += int64_t(a.tpr) * 8) {
                        uint32_t h[8];
                        pick8<RULE>(tab, a.idx, L, int64_t(r) * a.N + j, a.rows, h);
                        float w[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = f16_bits_to_f32(h[e]);
#pragma unroll
                        for (int t = 0; t < kRowsMaxTok; ++t)
                            if (uint32_t(t) < a.ntok) {
                                float xv[8];
                                load_x8<XDT>(a.X, (a.t0 + t) * a.N + j, xv);
#pragma unroll
                                for (int e = 0; e < 8; ++e) acc[t] += w[e] * xv[e];
                            }
                    }
                } else {
                    for (int64_t j = c; j < a.N; j += a.tpr) {
                        const float w = f16_bits_to_f32(pick<RULE>(tab, a.idx, L, int64_t(r) * a.N + j, a.rows));
#pragma unroll
                        for (int t = 0; t < kRowsMaxTok; ++t)
                            if (uint32_t(t) < a.ntok) acc[t] += w * load_elem<XDT>(a.X, (a.t0 + t) * a.N + j);
                    }
                }
            }
            for (uint32_t t = 0; t < a.ntok; ++t) red[t * kRowsThreads + threadIdx.x] = acc[t];
            __syncthreads();
            // thread (t, row) of the pass adds the row's tpr partial sums in order
            for (uint32_t u = threadIdx.x; u < a.ntok * rpp; u += kRowsThreads) {
                const uint32_t t = u / rpp, ro = u % rpp;
                if (r0 + ro < a.R) {
                    float s = 0.0f;
                    for (uint32_t k = 0; k < a.tpr; ++k) s += red[t * kRowsThreads + ro * a.tpr + k];
                    a.Y[(a.t0 + t) * a.M + b * a.R + r0 + ro] = ok ? s : __builtin_nanf("");
                }
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------------ GEMM (prefill)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
constexpr int kRBM = 128, kRBN = 128, kRBK = 32, kRLd = kRBK + 8;

struct RowsGemmArgs {
    const uint16_t* S;
    const uint16_t* idx;
    const ProjHeader* hdr;
    const uint16_t* X;   // [T][N] bf16 bits
    float* Y;
    int64_t T, M, N, nb;
    uint32_t R, Bg, seed, rows, tiles_m;
};

// 128 tokens x 128 outputs per workgroup (4 waves, 64 x 64 each as 2 x 2
// MFMA 32x32x16 bf16).  The tables of the tile's row blocks are staged in LDS;
// every 32-column K-chunk, X is copied to LDS and Ŵ is decoded into LDS (one
// gather per sketch row per weight, pick, binary16 -> bfloat16, exact for
// buckets of bfloat16 weights).
__global__ __launch_bounds__(256) void rows_gemm_kernel(RowsGemmArgs a, int rule) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    uint16_t* Xs = reinterpret_cast<uint16_t*>(lds_raw);   // [kRBM][kRLd]
    uint16_t* Ws = Xs + kRBM * kRLd;                        // [kRBN][kRLd]
    uint16_t* Ss = Ws + kRBN * kRLd;                        // tables of the tile's blocks
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t tile_m = blockIdx.x % a.tiles_m, tile_t = blockIdx.x / a.tiles_m;
    const int64_t o0 = tile_m * kRBN, t0 = tile_t * kRBM;
    const bool ok = rows_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed, a.rows);
    const int64_t L = int64_t(a.R) * a.N;

    const int64_t bA = o0 / a.R;
    int64_t bB = (o0 + kRBN - 1) / a.R;
    if (bB > a.nb - 1) bB = a.nb - 1;
    const int64_t nh = (bB - bA + 1) * int64_t(a.Bg);
    for (int64_t e = tid; e < nh; e += 256) Ss[e] = a.S[bA * a.Bg + e];

    const int o_d = tid >> 1, jseg = (tid & 1) * 16;
    const int64_t orow = o0 + o_d;
    const bool orow_ok = ok && orow < a.M;
    const uint32_t r_d = orow_ok ? uint32_t(orow % a.R) : 0;
    const uint16_t* Sblk = Ss + (orow_ok ? (orow / a.R - bA) * int64_t(a.Bg) : 0);
    const int x_r = tid >> 1, x_seg = (tid & 1) * 16;
    const int64_t xrow = t0 + x_r;
    const bool xrow_ok = xrow < a.T;
    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    float16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
    __syncthreads();

    for (int64_t j0 = 0; j0 < a.N; j0 += kRBK) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {   // X chunk -> LDS (N % 8 == 0)
            const int64_t j = j0 + x_seg + h * 8;
            uint4 v = {0, 0, 0, 0};
            if (xrow_ok && j < a.N) v = *reinterpret_cast<const uint4*>(a.X + xrow * a.N + j);
            *reinterpret_cast<uint4*>(Xs + x_r * kRLd + x_seg + h * 8) = v;
        }
        {   // Ŵ chunk -> LDS: two 8-column picks (N % 8 == 0)
            uint32_t pk[8];
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int64_t j = j0 + jseg + hh * 8;
                uint32_t h[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                if (orow_ok && j < a.N) {
                    if (rule == SKETCH_ABSMIN)
                        pick8<SKETCH_ABSMIN>(Sblk, a.idx, L, int64_t(r_d) * a.N + j, a.rows, h);
                    else
                        pick8<SKETCH_ABSMAX>(Sblk, a.idx, L, int64_t(r_d) * a.N + j, a.rows, h);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    pk[hh * 4 + e] = (__float_as_uint(f16_bits_to_f32(h[2 * e])) >> 16) |
                                     (__float_as_uint(f16_bits_to_f32(h[2 * e + 1])) & 0xFFFF0000u);
            }
            u32x4* dst = reinterpret_cast<u32x4*>(Ws + o_d * kRLd + jseg);
            dst[0] = u32x4{pk[0], pk[1], pk[2], pk[3]};
            dst[1] = u32x4{pk[4], pk[5], pk[6], pk[7]};
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kRBK / 16; ++ks) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(Xs + (wm + i * 32 + (lane & 31)) * kRLd + ks * 16 + (lane >> 5) * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(Ws + (wn + j * 32 + (lane & 31)) * kRLd + ks * 16 + (lane >> 5) * 8);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }
    // D[row][col]: row = 8*(v/4) + 4*(lane/32) + v%4, col = lane%32
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int64_t col = o0 + wn + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = t0 + wm + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < a.T && col < a.M) a.Y[row * a.M + col] = ok ? acc[i][j][v] : __builtin_nanf("");
            }
        }
}

inline int64_t rows_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu > 0 ? ncu : 256;
}

inline size_t rows_gemm_table_lds(const Shape& s) {
    const int64_t nblk = (kRBN - 1) / s.R + 2;
    return size_t(nblk < s.nb ? nblk : s.nb) * size_t(s.Bg) * 2;
}

}  // namespace

ProjLayout proj_layout_rows(int64_t R, int64_t N, int64_t rows) {
    ProjLayout L{};
    L.idx = align256(sizeof(ProjHeader));
    L.total = align256(L.idx + sizeof(uint16_t) * size_t(rows * R * N));
    L.off = L.cols = L.cnt = L.total;   // no inverse map: the product decodes every weight
    return L;
}

sketch_status launch_projection_build_rows(const sketch_params* p, const Shape& s, void* proj, hipStream_t st) {
    const ProjLayout L = proj_layout_rows(s.R, s.N, s.rows);
    char* base = static_cast<char*>(proj);
    ProjHeader h{kProjMagicRows, kProjVersion, uint32_t(s.R), uint32_t(s.N), uint32_t(s.Bg), p->seed,
                 {uint32_t(s.rows), 0}};
    const int64_t n = s.rows * s.R * s.N;
    rows_proj_kernel<<<unsigned((n + 255) / 256), 256, 0, st>>>(reinterpret_cast<ProjHeader*>(base), h,
                                                               reinterpret_cast<uint16_t*>(base + L.idx), s.R * s.N,
                                                               uint32_t(s.rows), uint32_t(s.Bg / s.rows), p->seed);
    return launch_status();
}

bool gemm_rows_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch) {
    return p->w_dtype == SKETCH_BF16 && xdt == SKETCH_BF16 && batch > kRowsMaxTok && s.N % 8 == 0 &&
           2 * kRBM * kRLd * 2 + rows_gemm_table_lds(s) <= 160 * 1024;
}

sketch_status launch_matmul_rows(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                                 const void* X, sketch_dtype xdt, int64_t batch, float* Y, hipStream_t st) {
    const char* pb = static_cast<const char*>(proj);
    const auto* idx = reinterpret_cast<const uint16_t*>(pb + proj_layout_rows(s.R, s.N, s.rows).idx);
    if (gemm_rows_supported(p, s, xdt, batch)) {
        RowsGemmArgs g;
        g.S = tables;
        g.idx = idx;
        g.hdr = static_cast<const ProjHeader*>(proj);
        g.X = static_cast<const uint16_t*>(X);
        g.Y = Y;
        g.T = batch;
        g.M = s.M;
        g.N = s.N;
        g.nb = s.nb;
        g.R = uint32_t(s.R);
        g.Bg = uint32_t(s.Bg);
        g.seed = p->seed;
        g.rows = uint32_t(s.rows);
        g.tiles_m = uint32_t((s.M + kRBN - 1) / kRBN);
        const int64_t grid = int64_t(g.tiles_m) * ((batch + kRBM - 1) / kRBM);
        if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
        const size_t lds = size_t(2 * kRBM * kRLd * 2) + ((rows_gemm_table_lds(s) + 15) & ~size_t(15));
        rows_gemm_kernel<<<unsigned(grid), 256, lds, st>>>(g, p->rule);
        return launch_status();
    }
    RowsGemvArgs a;
    a.S = tables;
    a.idx = idx;
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.X = X;
    a.Y = Y;
    a.M = s.M;
    a.N = s.N;
    a.nb = s.nb;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed = p->seed;
    a.rows = uint32_t(s.rows);
    // threads per weight row: a power of two, the rows of a pass fill the
    // workgroup; on the vector path no more threads than 8-column chunks
    const bool vec = s.N % 8 == 0;
    uint32_t tpr = kRowsThreads;
    while (tpr > 1 && tpr * uint32_t(s.R) > kRowsThreads) tpr >>= 1;
    while (vec && tpr > 1 && int64_t(tpr) * 8 > s.N) tpr >>= 1;
    a.tpr = tpr;
    const int64_t cap = 4 * rows_cus();
    const unsigned grid = unsigned(s.nb < cap ? s.nb : cap);
    const size_t lds = ((size_t(s.Bg) * 2 + 15) & ~size_t(15)) + size_t(kRowsMaxTok) * kRowsThreads * 4;
    for (int64_t t0 = 0; t0 < batch; t0 += kRowsMaxTok) {
        a.t0 = t0;
        a.ntok = uint32_t(batch - t0 < kRowsMaxTok ? batch - t0 : kRowsMaxTok);
#define SKETCH_ROWS_GEMV(XDT)                                                                             \
    (p->rule == SKETCH_ABSMIN                                                                             \
         ? (vec ? (rows_gemv_kernel<XDT, SKETCH_ABSMIN, true><<<grid, kRowsThreads, lds, st>>>(a), 0)       \
                : (rows_gemv_kernel<XDT, SKETCH_ABSMIN, false><<<grid, kRowsThreads, lds, st>>>(a), 0))     \
         : (vec ? (rows_gemv_kernel<XDT, SKETCH_ABSMAX, true><<<grid, kRowsThreads, lds, st>>>(a), 0)       \
                : (rows_gemv_kernel<XDT, SKETCH_ABSMAX, false><<<grid, kRowsThreads, lds, st>>>(a), 0)))
        switch (xdt) {
            case SKETCH_F32: SKETCH_ROWS_GEMV(SKETCH_F32); break;
            case SKETCH_BF16: SKETCH_ROWS_GEMV(SKETCH_BF16); break;
            default: SKETCH_ROWS_GEMV(SKETCH_F16); break;
        }
#undef SKETCH_ROWS_GEMV
        if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    }
    return SKETCH_OK;
}

}  // namespace sketch

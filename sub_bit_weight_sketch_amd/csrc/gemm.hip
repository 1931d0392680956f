// gemm.hip -- prefill product Y = X * W_hat^T with W_hat tiles decoded into LDS.
//
// "Resumen Técnico" › Metodología §4: decompression W_hat = S * P^T.  For a
// prefill batch the product is a dense contraction, so it runs on bf16 matrix
// cores: every output tile stages the bucket tables of its row blocks in LDS,
// decodes each K-chunk of W_hat from them through the projection's forward
// map, converts binary16 -> bfloat16 (exact for buckets of bfloat16 weights:
// every such binary16 value is a bfloat16 value), and accumulates in float32.
//
// Tile: 128 tokens x 128 outputs per workgroup (4 waves, each 64 x 64 as
// 2 x 2 MFMA 32x32x16 tiles), K-chunks of 32 columns.
#include "common.h"

namespace sketch {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kBM = 128;          // tokens per tile
constexpr int kBN = 128;          // outputs per tile
constexpr int kBK = 32;           // K-chunk
constexpr int kPad = 8;           // bf16 padding per LDS row
constexpr int kLdRow = kBK + kPad;
constexpr int kThreads = 256;
constexpr size_t kTableBudget = 96 * 1024;

struct GemmArgs {
    const uint16_t* S;     // [nb][Bg]
    const uint16_t* X;     // [T][N] bf16 bits
    const uint16_t* idx;   // forward map [R*N]
    const ProjHeader* hdr;
    float* Y;              // [T][M]
    int64_t T, M, N, nb;
    uint32_t R, Bg, seed_unused;
    uint32_t tiles_m;      // output tiles along M
};

__device__ inline uint16_t f16_to_bf16_exact(uint16_t h) {
    return uint16_t(__float_as_uint(f16_bits_to_f32(h)) >> 16);
}

__global__ __launch_bounds__(kThreads) void gemm_mfma_kernel(GemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    uint16_t* Xs = reinterpret_cast<uint16_t*>(lds_raw);            // [kBM][kLdRow]
    uint16_t* Ws = Xs + kBM * kLdRow;                                // [kBN][kLdRow]
    uint16_t* Ss = Ws + kBN * kLdRow;                                // [nblk][Bg]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t tile_m = blockIdx.x % a.tiles_m;   // output tile
    const int64_t tile_t = blockIdx.x / a.tiles_m;   // token tile
    const int64_t o0 = tile_m * kBN, t0 = tile_t * kBM;

    const bool ok = a.hdr->magic == kProjMagic && a.hdr->version == kProjVersion && a.hdr->R == a.R &&
                    a.hdr->N == uint32_t(a.N) && a.hdr->Bg == a.Bg;

    // Stage the bucket tables of blocks bA..bB.
    const int64_t bA = o0 / a.R;
    int64_t bB = (o0 + kBN - 1) / a.R;
    if (bB > a.nb - 1) bB = a.nb - 1;
    const int64_t nh = (bB - bA + 1) * int64_t(a.Bg);
    {
        const uint16_t* src = a.S + bA * int64_t(a.Bg);
        for (int64_t e = tid * 8; e < nh; e += kThreads * 8) {
            if (e + 8 <= nh) {
                *reinterpret_cast<uint4*>(Ss + e) = *reinterpret_cast<const uint4*>(src + e);
            } else {
                for (int64_t q = e; q < nh; ++q) Ss[q] = src[q];
            }
        }
    }

    // Per-thread decode assignment: output row o_d, 16 consecutive columns.
    const int o_d = tid >> 1, jseg = (tid & 1) * 16;
    const int64_t orow = o0 + o_d;
    const bool orow_ok = ok && orow < a.M;
    const uint32_t r_d = orow_ok ? uint32_t(orow % a.R) : 0;
    const uint16_t* Sblk = Ss + (orow_ok ? (orow / a.R - bA) * int64_t(a.Bg) : 0);
    const uint16_t* idx_row = a.idx + int64_t(r_d) * a.N;

    // Per-thread X assignment: row x_r, two 8-element segments.
    const int x_r = tid >> 1, x_seg = (tid & 1) * 16;
    const int64_t xrow = t0 + x_r;
    const bool xrow_ok = xrow < a.T;
    const uint16_t* xsrc = a.X + xrow * a.N;

    const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;
    float16v acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    __syncthreads();

    for (int64_t j0 = 0; j0 < a.N; j0 += kBK) {
        // X chunk -> LDS (N % 8 == 0 is a dispatch condition)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t j = j0 + x_seg + h * 8;
            uint4 v = {0, 0, 0, 0};
            if (xrow_ok && j < a.N) v = *reinterpret_cast<const uint4*>(xsrc + j);
            *reinterpret_cast<uint4*>(Xs + x_r * kLdRow + x_seg + h * 8) = v;
        }
        // decode W_hat chunk -> LDS
        {
            uint16_t out[16];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t j = j0 + jseg + h * 8;
                if (orow_ok && j < a.N) {
                    const uint4 kv = *reinterpret_cast<const uint4*>(idx_row + j);
                    const uint32_t ks[8] = {kv.x & 0xFFFFu, kv.x >> 16, kv.y & 0xFFFFu, kv.y >> 16,
                                            kv.z & 0xFFFFu, kv.z >> 16, kv.w & 0xFFFFu, kv.w >> 16};
#pragma unroll
                    for (int e = 0; e < 8; ++e) out[h * 8 + e] = f16_to_bf16_exact(Sblk[ks[e]]);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) out[h * 8 + e] = 0;
                }
            }
            uint4* dst = reinterpret_cast<uint4*>(Ws + o_d * kLdRow + jseg);
            dst[0] = make_uint4(out[0] | (uint32_t(out[1]) << 16), out[2] | (uint32_t(out[3]) << 16),
                                out[4] | (uint32_t(out[5]) << 16), out[6] | (uint32_t(out[7]) << 16));
            dst[1] = make_uint4(out[8] | (uint32_t(out[9]) << 16), out[10] | (uint32_t(out[11]) << 16),
                                out[12] | (uint32_t(out[13]) << 16), out[14] | (uint32_t(out[15]) << 16));
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            bf16x8 af[2], bfr[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                af[i] = *reinterpret_cast<const bf16x8*>(Xs + (wm + i * 32 + (lane & 31)) * kLdRow + ks * 16 +
                                                         (lane >> 5) * 8);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8*>(Ws + (wn + j * 32 + (lane & 31)) * kLdRow + ks * 16 +
                                                          (lane >> 5) * 8);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

    // Epilogue: D[row][col], row = 8*(v/4) + 4*(lane/32) + v%4, col = lane%32.
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

inline size_t table_lds(const Shape& s) {
    // worst case over tiles: blocks touched by 128 consecutive rows
    const int64_t nblk = (kBN - 1) / s.R + 2;
    const int64_t cap = nblk < s.nb ? nblk : s.nb;
    return size_t(cap) * size_t(s.Bg) * 2;
}

inline size_t lds_bytes(const Shape& s) { return size_t(2 * kBM * kLdRow * 2) + ((table_lds(s) + 15) & ~size_t(15)); }

}  // namespace

bool gemm_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch) {
    return p->w_dtype == SKETCH_BF16 && xdt == SKETCH_BF16 && batch > 16 && s.N % 8 == 0 && s.Bg % 8 == 0 &&
           table_lds(s) <= kTableBudget;
}

sketch_status launch_gemm(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                          const void* X, int64_t batch, float* Y, hipStream_t st) {
    (void)p;
    const ProjLayout L = proj_layout(s.R, s.N, s.Bg);
    GemmArgs a;
    a.S = tables;
    a.X = static_cast<const uint16_t*>(X);
    a.idx = reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + L.idx);
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.Y = Y;
    a.T = batch;
    a.M = s.M;
    a.N = s.N;
    a.nb = s.nb;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed_unused = 0;
    a.tiles_m = uint32_t((s.M + kBN - 1) / kBN);
    const int64_t tiles_t = (batch + kBM - 1) / kBM;
    const int64_t grid = int64_t(a.tiles_m) * tiles_t;
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    gemm_mfma_kernel<<<unsigned(grid), kThreads, lds_bytes(s), st>>>(a);
    return launch_status();
}

}  // namespace sketch

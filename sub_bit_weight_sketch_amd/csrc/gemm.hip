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
    uint32_t R, Bg, seed;
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
                    a.hdr->N == uint32_t(a.N) && a.hdr->Bg == a.Bg && a.hdr->seed == a.seed;

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

// ---------------------------------------------------------------------------
// gemm_tile_kernel<R, F>: 256 tokens x 32F outputs per workgroup, one
// workgroup per CU (4 waves, 32F float32 accumulators per lane).  F = 8 is
// the full tile; F = 7 (224 outputs, table words of 8 slots with one unused)
// gives whole rounds where 256-output tiles would leave a partial one (the
// 28672 outputs of the 70B MLP weight: 1024 tiles, 4 rounds, instead of 896
// tiles, 3.5 rounds); F = 4 is the half-width tile that evens out the last
// round of a launch of full tiles (see launch_gemm).
//
//  * Wave h owns tokens [64h, 64h+64) of the tile and all its outputs:
//    2 x F MFMA 32x32x16 bf16 tiles.  Every X element a wave loads feeds F
//    MFMAs, and no two waves load the same X.
//  * Ŵ columns come from the forward map: Ŵ[i][j] = S[i/R][k(r*N + j)] with
//    r = i % R.  In B fragment f (outputs 32f .. 32f+31) lane n holds output
//    32f + n, i.e. block f*Q + n/R and row n%R (Q = 32/R), so the F
//    fragments of a lane share one row r and therefore one index
//    k(r*N + j).  The LDS tables interleave those F blocks: one 2F-byte word
//    per (k, n/R) holds their F buckets, and one LDS read gathers a column
//    element for all F fragments.  Tables are converted to bfloat16 while
//    staged (exact for buckets of bfloat16 weights).
//  * After the tables are staged each wave loads its X fragments (A
//    operand) from global memory straight into registers, a group of 4
//    K-steps (64 columns) at a time and one group ahead: within a group the
//    k order is permuted so that a lane's 4 loads cover 64 contiguous bytes
//    of its token row.  The forward map is copied into LDS 256 columns at a
//    time (double-buffered, in the same permuted order, one barrier per
//    chunk).  Step s gathers the table words of step s+2 and unpacks the
//    words of step s+1 (gathered a step ago) into B fragments, so nothing it
//    issues waits on an LDS read of its own.
// ---------------------------------------------------------------------------
constexpr int kT2 = 256;             // tokens per tile
constexpr int kKS = 16;              // K-step
constexpr int kGroup = 4;            // K-steps whose X one lane loads as 64 contiguous bytes
constexpr int kChunk = 16;           // K-steps per forward-map chunk in LDS (256 columns)

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int F> struct TableWord;
template <> struct TableWord<8> { typedef u32x4 type; };
template <> struct TableWord<4> { typedef u32x2 type; };
template <> struct TableWord<7> { typedef u32x4 type; };   // 8 slots, the last one unused

// Blocks a table word holds: F, or 8 for the 7-fragment tile.
template <int F> constexpr int word_slots() { return F == 7 ? 8 : F; }

struct Gemm2Args {
    const uint16_t* S;     // [nb][Bg] binary16 (4-bit sketch: the packed codes, [nb][Bg/2] bytes)
    const uint16_t* scales;   // 4-bit sketch: binary16 scale per block
    const uint16_t* X;     // [T][N] bf16 bits
    const uint16_t* idx;   // forward map [R*N]
    const ProjHeader* hdr;
    float* Y;              // [T][M]
    int64_t T, M, N, nb;
    uint32_t R, Bg, Q;     // Q = 32 / R
    uint32_t seed;
    uint32_t tiles_o;      // output tiles (32F outputs) per token tile
    uint32_t tile0;        // linear index (token tile major) of the launch's first tile
};

__device__ inline uint32_t bf16_pair(uint32_t a_lo, uint32_t b_hi) { return a_lo | (b_hi << 16); }

// Direct global->LDS load of 16 bytes per lane: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16).  `lds` is the wave-uniform LDS byte address.
// Written as inline asm on purpose: the compiler treats the builtin's LDS
// write as aliasing every LDS access and waits for all outstanding loads
// before each of them; here the one wait that matters is explicit.  The
// instruction has no register result; M0 needs one wait state after its
// write.
__device__ inline void dma16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds) : "memory", "m0");
}

// LDS of one forward-map chunk: kChunk steps x R rows x 32 bytes, at least
// one 256-thread round of 16-byte pieces.
__host__ __device__ constexpr uint32_t chunk_bytes(uint32_t R) {
    const uint32_t b = uint32_t(kChunk) * R * 32;
    return b > 4096u ? b : 4096u;
}

// base + stride * (16-bit half HI of packed): one v_mad_u32_u16 whose op_sel
// picks the half, where the compiler would first mask or shift the half out
// and then multiply-add (two instructions per gathered column).  A plain
// VALU instruction: no memory access, no wait.
template <int HI>
__device__ inline uint32_t mad_half(uint32_t packed, uint32_t stride, uint32_t base) {
    uint32_t d;
    if (HI)
        asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(d) : "v"(packed), "s"(stride), "v"(base));
    else
        asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(d) : "v"(packed), "s"(stride), "v"(base));
    return d;
}

__device__ inline uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}

// R (rows per block, a power of two up to 32) is a template parameter so
// that every per-step offset is an immediate.  Q4: a 4-bit sketch (codes q
// in [-7, 7], one binary16 scale s per block, W_hat = q * s with the same
// hash as binary16 buckets): the codes are staged as bfloat16 words (exact
// small integers) and each output is scaled by its block's s in the
// epilogue.
template <int R, int F, bool Q4>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_tile_kernel(Gemm2Args a) {
    static_assert(F == 8 || F == 7 || F == 4, "table words hold 8 (7 used) or 4 blocks");
    constexpr int FW = word_slots<F>();
    static_assert(R >= 1 && R <= 32 && (R & (R - 1)) == 0, "R is a power of two up to 32");
    typedef typename TableWord<F>::type word_t;
    constexpr int kO = 32 * F;                 // outputs per tile
    constexpr uint32_t Q = 32 / R;             // blocks per fragment
    constexpr uint32_t lgR = __builtin_ctz(R), lgQ = 5 - lgR;
    constexpr int PPT = R <= 8 ? 1 : R / 8;    // 16-byte forward-map pieces per thread and chunk
    constexpr uint32_t cbytes = chunk_bytes(R);
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const uint32_t Bg = a.Bg;
    unsigned char* ichunk = lds;                                        // [2][kChunk][R][2][8] u16
    unsigned char* tab = lds + 2 * size_t(chunk_bytes(R));              // [Bg][Q] x 2F bytes

    const int tid = threadIdx.x, lane = tid & 63;
    const int h = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-aware order: consecutive workgroups of one XCD share a token tile
    uint32_t bid = blockIdx.x;
    if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
    bid += a.tile0;
    const uint32_t tile_o = bid % a.tiles_o, tile_t = bid / a.tiles_o;
    const int64_t o0 = int64_t(tile_o) * kO, t0 = int64_t(tile_t) * kT2;
    const int64_t b0 = o0 / R;
    const uint32_t nsteps = uint32_t(a.N / kKS);

    const uint4 h0 = reinterpret_cast<const uint4*>(a.hdr)[0];
    const uint4 h1 = reinterpret_cast<const uint4*>(a.hdr)[1];
    const bool ok = h0.x == kProjMagic && h0.y == kProjVersion && h0.z == uint32_t(R) && h0.w == uint32_t(a.N) &&
                    h1.x == a.Bg && h1.y == a.seed;
    // A projection built for other parameters: the tile's outputs are NaN and
    // its forward map is never read (the branch is uniform).
    if (!ok) {
        for (uint32_t u = tid; u < uint32_t(kT2 * kO); u += 256) {
            const int64_t t = t0 + u / kO, o = o0 + u % kO;
            if (t < a.T && o < a.M) a.Y[t * a.M + o] = __builtin_nanf("");
        }
        return;
    }

    // ---- tables of the tile's blocks -> LDS as bf16 words of F blocks.
    // Unit (q, kb): 8 consecutive k of blocks b0 + f*Q + q, f < F, read as F
    // rows of 16 bytes and written as the 8 words (k, q).
    {
        const uint32_t units = Q * (Bg / 8);
        for (uint32_t un = tid; un < units; un += 256) {
            const uint32_t q = un & (Q - 1), kb = un >> lgQ;
            uint32_t v[F][4];
#pragma unroll
            for (int f = 0; f < F; ++f) {
                const int64_t blk = b0 + int64_t(f) * Q + q;
                if constexpr (Q4) {   // 8 codes: 4 bytes, the even bucket in the low nibble
                    v[f][0] = blk < a.nb ? *reinterpret_cast<const uint32_t*>(
                                               reinterpret_cast<const uint8_t*>(a.S) + blk * (Bg / 2) + kb * 4)
                                         : 0u;
                } else {
                    uint4 raw = {0, 0, 0, 0};
                    if (blk < a.nb) raw = *reinterpret_cast<const uint4*>(a.S + blk * Bg + kb * 8);
                    v[f][0] = raw.x; v[f][1] = raw.y; v[f][2] = raw.z; v[f][3] = raw.w;
                }
            }
            // bfloat16 bits of bucket k = 8 kb + e of fragment f's block
            auto bucket_bf16 = [&](int f, int e) -> uint32_t {
                if constexpr (Q4) {
                    const int code = int((v[f][0] >> (4 * e)) << 28) >> 28;
                    return __float_as_uint(float(code)) >> 16;
                } else {
                    return __float_as_uint(f16_bits_to_f32((v[f][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu)) >> 16;
                }
            };
#pragma unroll
            for (int e = 0; e < 8; ++e) {   // k = 8 kb + e
                word_t wv;
#pragma unroll
                for (int d = 0; d < FW / 2; ++d)
                    wv[d] = bf16_pair(bucket_bf16(2 * d, e), 2 * d + 1 < F ? bucket_bf16(2 * d + 1, e) : 0u);
                *reinterpret_cast<word_t*>(tab + (size_t(kb * 8 + e) * Q + q) * (2 * FW)) = wv;
            }
        }
    }

    __syncthreads();   // tables staged

    const uint32_t n = lane & 31, kh = lane >> 5;
    // X fragment i: token h*64 + i*32 + n.  Within a group of 4 K-steps (64
    // columns) the k order is permuted: at step u of the group, lane half kh
    // holds columns kh*32 + u*8 .. +8, so the 4 loads of one fragment read 64
    // contiguous bytes of its token row.  The forward-map slices are staged
    // in the same order.
    const uint16_t* xrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        int64_t t = t0 + h * 64 + i * 32 + n;
        t = t < a.T ? t : a.T - 1;
        xrow[i] = a.X + t * a.N + kh * 32;
    }
    const uint32_t ngroups = nsteps / kGroup;
    auto load_group = [&](uint32_t G, bf16x8 (&xg)[2][4]) {
        const int64_t col = int64_t(G < ngroups ? G : ngroups - 1) * (kGroup * kKS);
#pragma unroll
        for (int o = 0; o < 8; ++o) {
            const int i = o >> 2, u = o & 3;
            xg[i][u] = *reinterpret_cast<const bf16x8*>(xrow[i] + col + u * 8);
        }
    };
    // Forward map, chunk c = columns [256c, 256c + 256), staged in LDS as
    // [step j][row][half][8] u16 (R * 512 bytes); the whole workgroup shares
    // it.  Piece p = (j, row, half) of 16 bytes is copied by thread p % 256.
    const uint32_t nchunks = nsteps / kChunk;
    const uint32_t ichunk_a = lds_addr(ichunk);
    const uint32_t npieces = uint32_t(kChunk) * R * 2;          // 16-byte pieces per chunk
    auto issue_chunk = [&](uint32_t c, uint32_t buf) {
        const uint32_t src_c = c < nchunks ? c : nchunks - 1;
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            // threads past the last piece copy it again into the padding
            // (cbytes >= 4 KiB), so every wave issues the same instructions
            const uint32_t p0 = uint32_t(k) * 256;
            const uint32_t pc = p0 + uint32_t(tid) < npieces ? p0 + uint32_t(tid) : npieces - 1;
            const uint32_t j = pc >> (lgR + 1), rr = (pc >> 1) & (R - 1), hf = pc & 1;
            dma16(a.idx + int64_t(rr) * a.N + int64_t(src_c) * (kChunk * kKS) + (j >> 2) * 64 + hf * 32 + (j & 3) * 8,
                  ichunk_a + buf * cbytes + p0 * 16 + uint32_t(h) * 64 * 16);
        }
    };
    const uint32_t r = n & (R - 1), q = n >> lgR;
    const uint32_t ioff = (r * 2 + kh) * 16;
    auto read_idx = [&](uint32_t st) {
        const uint32_t buf = (st / kChunk) & 1u, j = st % kChunk;
        return *reinterpret_cast<const u32x4*>(ichunk + buf * cbytes + j * (R * 32) + ioff);
    };

    // Gathers of a step: the slice gives 8 column indices; one table word
    // per column holds the element for all F fragments.
    typedef const __attribute__((address_space(3))) word_t* lds_word_ptr;
    const uint32_t tab_q = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tab + q * (2 * FW)));
    const uint32_t wstride = Q * (2 * FW);   // bytes per k
    auto gather_words = [&](const u32x4 iv, word_t (&w)[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t addr = (e & 1) ? mad_half<1>(iv[e >> 1], wstride, tab_q) : mad_half<0>(iv[e >> 1], wstride, tab_q);
            w[e] = *reinterpret_cast<lds_word_ptr>(addr);
        }
    };
    // word dword d = (fragment 2d, fragment 2d + 1); column pair (2p, 2p + 1)
    auto unpack = [&](const word_t (&w)[8], bf16x8 (&bf)[F]) {
#pragma unroll
        for (int p = 0; p < 4; ++p)
#pragma unroll
            for (int d = 0; d < FW / 2; ++d) {
                reinterpret_cast<uint32_t*>(&bf[2 * d])[p] = __builtin_amdgcn_perm(w[2 * p + 1][d], w[2 * p][d], 0x05040100u);
                if (2 * d + 1 < F)
                    reinterpret_cast<uint32_t*>(&bf[2 * d + 1])[p] =
                        __builtin_amdgcn_perm(w[2 * p + 1][d], w[2 * p][d], 0x07060302u);
            }
    };

    float16v acc[2][F];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

    // Prologue: chunk 0 of the forward map, B fragments of step 0, the
    // table words of step 1, the slice of step 2 and the X of group 0.
    bf16x8 xa[2][4], xb[2][4];
    bf16x8 bA[F], bB[F];
    word_t wA[8], wB[8];
    u32x4 ivA, ivB;
    issue_chunk(0, 0);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    {
        word_t w0[8];
        gather_words(read_idx(0), w0);
        unpack(w0, bA);                        // B fragments of step 0
        gather_words(read_idx(1), wA);         // words of step 1
        ivA = read_idx(2);
    }
    load_group(0, xa);

    // One K-step s (step u of its group): gather step s+2's table words with
    // the slice read a step ago, read step s+3's slice, unpack step s+1's
    // words (gathered a step ago) into its B fragments and run the 2F MFMAs
    // of step s; at u == 0 also load the X of the next group into the other
    // buffer (consumed by the previous step).  The scheduling groups spread
    // the gathers, the loads and the unpacking between the MFMAs so that the
    // matrix core never waits for the single wave of its SIMD to issue them.
    auto step = [&](uint32_t s, const int u, const bf16x8 (&xg)[2][4], bf16x8 (&xn)[2][4], const bf16x8 (&bc)[F],
                    bf16x8 (&bn)[F], const word_t (&wn)[8], word_t (&wnn)[8], const u32x4 ivc, u32x4& ivn) {
        // the slice goes out first: the next step waits only for it, and
        // LDS reads complete in order.  Past the last step it reads the
        // extra copy of the last chunk (see issue_chunk): valid indices,
        // unused results.
        ivn = read_idx(s + 3);
        gather_words(ivc, wnn);
        unpack(wn, bn);
#pragma unroll
        for (int f = 0; f < F; ++f)
#pragma unroll
            for (int i = 0; i < 2; ++i)
                acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xg[i][u], bc[f], acc[i][f], 0, 0, 0);
        if (u == 0) load_group(s / kGroup + 1, xn);
        // per MFMA: the 9 LDS reads and the loads go with the first ones,
        // the 4F + 8 VALU are spread over all 2F
        constexpr int kV = (4 * F + 8 + 2 * F - 1) / (2 * F);
#pragma unroll
        for (int k = 0; k < 2 * F; ++k) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if (k < 9) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            if (u == 0 && k < 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
        }
        __builtin_amdgcn_sched_barrier(0);   // steps are scheduled one at a time
    };
    static_assert(kGroup == 4 && kChunk == 4 * kGroup, "the loop below runs 4 groups per chunk, 2 X buffers");

    // Chunk c+1 is requested after step 1 of chunk c (its buffer last held
    // chunk c-1, whose final slice was read at step 12 of chunk c-1, before
    // the barrier that follows that step), and must have landed before step
    // 13 of chunk c, which reads the first slice of chunk c+1.  Between the
    // request and that barrier the wave issues the X loads of steps 4, 8 and
    // 12 (8 each; nothing else touches vmcnt), so "vmcnt(24)" waits for the
    // chunk only.  One barrier per chunk.
    for (uint32_t c = 0; c < nchunks; ++c) {
        const uint32_t s0 = c * kChunk;
#pragma unroll
        for (uint32_t j = 0; j < kChunk; j += 2 * kGroup) {
            step(s0 + j, 0, xa, xb, bA, bB, wA, wB, ivA, ivB);
            step(s0 + j + 1, 1, xa, xb, bB, bA, wB, wA, ivB, ivA);
            if (j == 0) issue_chunk(c + 1, (c + 1) & 1u);
            step(s0 + j + 2, 2, xa, xb, bA, bB, wA, wB, ivA, ivB);
            step(s0 + j + 3, 3, xa, xb, bB, bA, wB, wA, ivB, ivA);
            step(s0 + j + 4, 0, xb, xa, bA, bB, wA, wB, ivA, ivB);
            if (j + 2 * kGroup == kChunk) asm volatile("s_waitcnt vmcnt(24)\n\ts_barrier" ::: "memory");
            step(s0 + j + 5, 1, xb, xa, bB, bA, wB, wA, ivB, ivA);
            step(s0 + j + 6, 2, xb, xa, bA, bB, wA, wB, ivA, ivB);
            step(s0 + j + 7, 3, xb, xa, bB, bA, wB, wA, ivB, ivA);
        }
    }

    // ---- epilogue: D[m][n] with m = 8*(v/4) + 4*(lane/32) + v%4, n = lane%32
    const int64_t trow = t0 + h * 64 + 4 * kh;       // token of m = 0 in this lane
    const int64_t ocol = o0 + n;                     // output of fragment 0
    float* ybase = a.Y + trow * a.M + ocol;
    float osc[F];                                    // 4-bit sketch: scale of each fragment's block
#pragma unroll
    for (int f = 0; f < F; ++f) {
        osc[f] = 1.0f;
        if constexpr (Q4) {
            const int64_t o = ocol + f * 32;
            if (o < a.M) osc[f] = f16_bits_to_f32(a.scales[o / R]);
        }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = i * 32 + 8 * (v >> 2) + (v & 3);
            if (trow + m < a.T) {
#pragma unroll
                for (int f = 0; f < F; ++f)
                    if (ocol + f * 32 < a.M) {
                        const float y = Q4 ? acc[i][f][v] * osc[f] : acc[i][f][v];
                        __builtin_nontemporal_store(y, ybase + m * a.M + f * 32);
                    }
            }
        }
}

// LDS of a tile with F fragments per wave: two forward-map chunks and the
// tables of 32F outputs (32F / R blocks of Bg bf16 buckets).
inline size_t tile_lds(const Shape& s, int F) {
    const int FW = F == 7 ? 8 : F;
    return 2 * size_t(chunk_bytes(uint32_t(s.R))) + size_t(32 * FW / s.R) * s.Bg * 2;
}

inline bool tile_supported(const Shape& s) {
    const bool pow2R = s.R > 0 && (s.R & (s.R - 1)) == 0;
    return pow2R && s.R <= 32 && s.N % (kKS * kChunk) == 0 && s.Bg % 8 == 0 && tile_lds(s, 8) <= 160 * 1024;
}

// Compute units of the current device (cached per device).
inline int64_t device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int ncu = 256;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || ncu <= 0) ncu = 256;
    if (dev < 64) cached[dev] = ncu;
    return ncu;
}

constexpr size_t kHalfTileLds = 81 * 1024;   // > 80 KiB: at most one workgroup per CU

template <int F, bool Q4 = false>
sketch_status launch_tile(const Gemm2Args& b, unsigned grid, size_t lds, hipStream_t st) {
    switch (b.R) {
        case 1: gemm_tile_kernel<1, F, Q4><<<grid, 256, lds, st>>>(b); break;
        case 2: gemm_tile_kernel<2, F, Q4><<<grid, 256, lds, st>>>(b); break;
        case 4: gemm_tile_kernel<4, F, Q4><<<grid, 256, lds, st>>>(b); break;
        case 8: gemm_tile_kernel<8, F, Q4><<<grid, 256, lds, st>>>(b); break;
        case 16: gemm_tile_kernel<16, F, Q4><<<grid, 256, lds, st>>>(b); break;
        case 32: gemm_tile_kernel<32, F, Q4><<<grid, 256, lds, st>>>(b); break;
        default: return SKETCH_EINVAL;
    }
    return launch_status();
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
    return p->w_dtype == SKETCH_BF16 && xdt == SKETCH_BF16 && batch > 16 &&
           (tile_supported(s) || (s.N % 8 == 0 && s.Bg % 8 == 0 && table_lds(s) <= kTableBudget));
}

sketch_status launch_gemm(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                          const void* X, int64_t batch, float* Y, hipStream_t st) {
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
    a.seed = p->seed;
    if (tile_supported(s)) {
        Gemm2Args b;
        b.S = tables;
        b.X = static_cast<const uint16_t*>(X);
        b.idx = reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + L.idx);
        b.hdr = static_cast<const ProjHeader*>(proj);
        b.Y = Y;
        b.T = batch;
        b.M = s.M;
        b.N = s.N;
        b.nb = s.nb;
        b.R = uint32_t(s.R);
        b.Bg = uint32_t(s.Bg);
        b.Q = 32u / uint32_t(s.R);
        b.seed = p->seed;
        b.scales = nullptr;
        // Each CU holds one 256 x 256 tile at a time.  When the last round
        // of tiles would fill at most half the CUs, the whole rounds run as
        // 256 x 256 tiles and the remaining tiles as twice as many 256 x 128
        // tiles, so the last round takes about half as long.
        const int64_t tiles_o = (s.M + 255) / 256;
        const int64_t tiles_t = (batch + kT2 - 1) / kT2;
        const int64_t tiles = tiles_o * tiles_t;
        if (tiles > 0x3FFFFFFF) return SKETCH_EINVAL;
        const int64_t ncu = device_cus();
        const int64_t rem = tiles % ncu;
        const int64_t full = rem > 0 && 2 * rem <= ncu ? tiles - rem : tiles;
        // Rounds of work in units of a 256 x 256 tile round: whole rounds of
        // 256 x 256 tiles plus a round of half-width tiles (about 0.72 of a
        // full round), against whole rounds of 256 x 224 tiles (7/8 of the
        // work each, taken 4% less efficient).
        const double cost8 = full < tiles ? double(full / ncu) + 0.72 : double((tiles + ncu - 1) / ncu);
        const int64_t tiles_o7 = (s.M + 223) / 224, tiles7 = tiles_o7 * tiles_t;
        const double cost7 = double((tiles7 + ncu - 1) / ncu) * 0.875 * 1.04;
        if (cost7 < cost8 && tiles7 <= 0x3FFFFFFF) {
            b.tiles_o = uint32_t(tiles_o7);
            b.tile0 = 0;
            return launch_tile<7>(b, unsigned(tiles7), tile_lds(s, 7), st);
        }
        if (full > 0) {
            b.tiles_o = uint32_t(tiles_o);
            b.tile0 = 0;
            if (launch_tile<8>(b, unsigned(full), tile_lds(s, 8), st) != SKETCH_OK) return SKETCH_EDEVICE;
        }
        if (full < tiles) {
            // half-width tiles: 2 per 256-wide tile (the second half of a
            // ragged last tile may hold no outputs); dynamic LDS above half a
            // CU keeps them one per CU
            b.tiles_o = uint32_t(2 * tiles_o);
            b.tile0 = uint32_t(2 * full);
            size_t lds = tile_lds(s, 4);
            if (lds < kHalfTileLds) lds = kHalfTileLds;
            if (launch_tile<4>(b, unsigned(2 * (tiles - full)), lds, st) != SKETCH_OK) return SKETCH_EDEVICE;
        }
        return SKETCH_OK;
    }
    a.tiles_m = uint32_t((s.M + kBN - 1) / kBN);
    const int64_t tiles_t = (batch + kBM - 1) / kBM;
    const int64_t grid = int64_t(a.tiles_m) * tiles_t;
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    gemm_mfma_kernel<<<unsigned(grid), kThreads, lds_bytes(s), st>>>(a);
    return launch_status();
}

// 4-bit sketch on the tile kernel: Bg is the 4-bit bucket count, tables the
// packed codes with the scales at `scales`.  Its tables are four times those
// of binary16 buckets at the same bpw, so every tile is the 256 x 128 one.
bool gemm_tile_q4_supported(const Shape& s, sketch_dtype xdt, int64_t batch) {
    const bool pow2R = s.R > 0 && (s.R & (s.R - 1)) == 0;
    return xdt == SKETCH_BF16 && batch > 16 && pow2R && s.R <= 32 && s.N % (kKS * kChunk) == 0 && s.Bg % 8 == 0 &&
           tile_lds(s, 4) <= 160 * 1024;
}

sketch_status launch_gemm_tile_q4(const sketch_params* p, const Shape& s, const void* proj, const uint8_t* codes,
                                  const uint16_t* scales, const void* X, int64_t batch, float* Y, hipStream_t st) {
    const ProjLayout L = proj_layout(s.R, s.N, s.Bg);
    Gemm2Args b;
    b.S = reinterpret_cast<const uint16_t*>(codes);
    b.scales = scales;
    b.X = static_cast<const uint16_t*>(X);
    b.idx = reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + L.idx);
    b.hdr = static_cast<const ProjHeader*>(proj);
    b.Y = Y;
    b.T = batch;
    b.M = s.M;
    b.N = s.N;
    b.nb = s.nb;
    b.R = uint32_t(s.R);
    b.Bg = uint32_t(s.Bg);
    b.Q = 32u / uint32_t(s.R);
    b.seed = p->seed;
    const int64_t tiles_o = (s.M + 127) / 128;
    const int64_t tiles = tiles_o * ((batch + kT2 - 1) / kT2);
    if (tiles > 0x3FFFFFFF) return SKETCH_EINVAL;
    b.tiles_o = uint32_t(tiles_o);
    b.tile0 = 0;
    size_t lds = tile_lds(s, 4);
    if (lds < kHalfTileLds) lds = kHalfTileLds;
    return launch_tile<4, true>(b, unsigned(tiles), lds, st);
}

}  // namespace sketch

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

// ---------------------------------------------------------------------------
// gemm_tile_kernel: 256 tokens x 256 outputs per workgroup, one workgroup per
// CU (4 waves, 256 float32 accumulators each).
//
//  * Wave (g, h) = (wave & 1, wave >> 1) owns outputs [128g, 128g+128) and
//    tokens [128h, 128h+128) of the tile: 4 x 4 MFMA 32x32x16 bf16 tiles.
//  * Ŵ columns come from the forward map: Ŵ[i][j] = S[i/R][k(r*N + j)] with
//    r = i % R.  In a B fragment (32 outputs) lane n holds output f*32 + n
//    of its group, i.e. block f*Q + n/R and row n%R (Q = 32/R), so the 4
//    fragments of a lane share one row r and therefore one index
//    k(r*N + j).  The LDS tables interleave those 4 blocks: one 8-byte word
//    per (group, n/R, k) holds the 4 buckets, and one ds_read_b64 gathers a
//    column element for all 4 fragments.  Tables are converted to bfloat16
//    while staged (exact for buckets of bfloat16 weights).
//  * Every K-step (16 columns) streams through LDS with direct global->LDS
//    loads: X as [256 tokens][16] bf16 (8 KiB, three buffers, two steps
//    ahead, shared by the workgroup) and the forward-map slice of the step
//    as [R rows][16] u16 (three buffers per wave, three steps ahead, private
//    to the wave).  One barrier per step; the B fragments of step s+1 are
//    gathered while step s multiplies.
// ---------------------------------------------------------------------------
constexpr int kT2 = 256;             // tokens per tile
constexpr int kO2 = 256;             // outputs per tile
constexpr int kKS = 16;              // K-step
constexpr int kRing = 3;             // buffers per staged stream
constexpr size_t kXStepBytes = size_t(kT2) * kKS * 2;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct Gemm2Args {
    const uint16_t* S;     // [nb][Bg] binary16
    const uint16_t* X;     // [T][N] bf16 bits
    const uint16_t* idx;   // forward map [R*N]
    const ProjHeader* hdr;
    float* Y;              // [T][M]
    int64_t T, M, N, nb;
    uint32_t R, Bg, Q;     // Q = 32 / R
    uint32_t tiles_o;      // output tiles
};

__device__ inline uint32_t bf16_pair(uint32_t a_lo, uint32_t b_hi) { return a_lo | (b_hi << 16); }

// Direct global->LDS load of 16 bytes per lane: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16).  `lds` is the wave-uniform LDS byte address.
// Written as inline asm on purpose: the compiler treats the builtin's LDS
// write as aliasing every LDS access and waits for all outstanding loads
// before each of them, which serialises the ring buffers below; here the
// waits are explicit (s_waitcnt vmcnt before the barrier of each step).
// The instruction has no register result; M0 needs one wait state after
// its write.
__device__ inline void dma16(const void* src, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(lds)
                 : "memory", "m0");
}

__device__ inline uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p)));
}

__host__ __device__ inline size_t idx_ring_bytes(uint32_t R) { return size_t(kRing) * 2 * R * 16; }   // per wave

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_tile_kernel(Gemm2Args a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const uint32_t Q = a.Q, Bg = a.Bg, R = a.R;
    unsigned char* xbuf = lds;                                          // [kRing][kT2][16] bf16
    unsigned char* ibuf = lds + kRing * kXStepBytes;                    // [4 waves][kRing][R][2][8] u16
    unsigned char* tab = ibuf + 4 * idx_ring_bytes(R);                  // [2][Q][Bg] x 8 bytes

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = wave & 1, h = wave >> 1;
    // XCD-aware order: consecutive workgroups of one XCD share an output tile
    uint32_t bid = blockIdx.x;
    if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
    const uint32_t tile_o = bid % a.tiles_o, tile_t = bid / a.tiles_o;
    const int64_t o0 = int64_t(tile_o) * kO2, t0 = int64_t(tile_t) * kT2;
    const int64_t b0 = o0 / R;
    const uint32_t nsteps = uint32_t(a.N / kKS);

    const uint4 h0 = reinterpret_cast<const uint4*>(a.hdr)[0];
    const uint4 h1 = reinterpret_cast<const uint4*>(a.hdr)[1];
    const bool ok = h0.x == kProjMagic && h0.y == kProjVersion && h0.z == a.R && h0.w == uint32_t(a.N) && h1.x == a.Bg;

    // ---- staged streams.  X chunk c of a step = (token c/2, half c%2).
    unsigned char* wibuf = ibuf + size_t(wave) * idx_ring_bytes(R);
    const uint32_t ic = uint32_t(lane) < 2 * R ? uint32_t(lane) : 2 * R - 1;   // (row ic/2, half ic%2)
    const uint16_t* isrc = a.idx + int64_t(ic >> 1) * a.N + (ic & 1) * 8;
    const uint32_t xbuf_a = lds_addr(xbuf), wibuf_a = lds_addr(wibuf);
    auto issue = [&](uint32_t xstep, uint32_t istep) {
        const uint32_t dst = xbuf_a + (xstep % kRing) * uint32_t(kXStepBytes);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t c = uint32_t(i * 256 + tid);
            int64_t t = t0 + (c >> 1);
            t = t < a.T ? t : a.T - 1;
            const uint16_t* src = a.X + t * a.N + int64_t(xstep) * kKS + (c & 1) * 8;
            dma16(src, dst + uint32_t(i * 256 + wave * 64) * 16);
        }
        if (uint32_t(lane) < 2 * R) dma16(isrc + int64_t(istep) * kKS, wibuf_a + (istep % kRing) * (2 * R * 16));
    };
    auto clampstep = [&](uint32_t st) { return st < nsteps ? st : nsteps - 1; };

    // ---- tables of the tile's blocks -> LDS, interleaved by 4, as bf16
    {
        const uint32_t words = 2 * Q * Bg;   // (g, q, k)
        for (uint32_t w8 = tid * 8; w8 < words; w8 += 256 * 8) {
            // 8 consecutive k of one (g, q): Bg % 8 == 0
            const uint32_t gq = w8 / Bg, k = w8 % Bg;
            const uint32_t gg = gq / Q, q = gq % Q;
            uint32_t v[4][4];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int64_t blk = b0 + int64_t(gg) * (128 / R) + f * Q + q;
                uint4 raw = {0, 0, 0, 0};
                if (blk < a.nb) raw = *reinterpret_cast<const uint4*>(a.S + blk * Bg + k);
                v[f][0] = raw.x; v[f][1] = raw.y; v[f][2] = raw.z; v[f][3] = raw.w;
            }
            u32x4* dst = reinterpret_cast<u32x4*>(tab + size_t(w8) * 8);
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {   // k pairs (2 e2, 2 e2 + 1)
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    lo[f] = __float_as_uint(f16_bits_to_f32(v[f][e2] & 0xFFFFu)) >> 16;
                    hi[f] = __float_as_uint(f16_bits_to_f32(v[f][e2] >> 16)) >> 16;
                }
                dst[e2] = u32x4{bf16_pair(lo[0], lo[1]), bf16_pair(lo[2], lo[3]), bf16_pair(hi[0], hi[1]),
                                bf16_pair(hi[2], hi[3])};
            }
        }
    }
    // prologue streams: X of steps 0, 1 and forward-map slices of steps 0, 1, 2
    issue(0, 0);
    issue(clampstep(1), clampstep(1));
    if (uint32_t(lane) < 2 * R) dma16(isrc + int64_t(clampstep(2)) * kKS, wibuf_a + (clampstep(2) % kRing) * (2 * R * 16));
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- per-lane gather addresses
    const uint32_t n = lane & 31, kh = lane >> 5;
    const uint32_t r = n % R, q = n / R;
    const uint32_t tbase = (uint32_t(g) * Q + q) * Bg;   // word index of (g, q, 0)
    const u32x2* tab64 = reinterpret_cast<const u32x2*>(tab);
    const uint32_t ioff = (r * 2 + kh) * 16;

    float16v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.0f;

    // B fragments of step t from its forward-map slice (wave-private ring)
    auto gather = [&](uint32_t t, bf16x8 (&bf)[4]) {
        const u32x4 iv = *reinterpret_cast<const u32x4*>(wibuf + (t % kRing) * (2 * R * 16) + ioff);
        u32x2 w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t kk = (iv[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
            w[e] = tab64[tbase + kk];
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            // word lo = (f0, f1), hi = (f2, f3); column pair (2p, 2p + 1)
            reinterpret_cast<uint32_t*>(&bf[0])[p] = __builtin_amdgcn_perm(w[2 * p + 1].x, w[2 * p].x, 0x05040100u);
            reinterpret_cast<uint32_t*>(&bf[1])[p] = __builtin_amdgcn_perm(w[2 * p + 1].x, w[2 * p].x, 0x07060302u);
            reinterpret_cast<uint32_t*>(&bf[2])[p] = __builtin_amdgcn_perm(w[2 * p + 1].y, w[2 * p].y, 0x05040100u);
            reinterpret_cast<uint32_t*>(&bf[3])[p] = __builtin_amdgcn_perm(w[2 * p + 1].y, w[2 * p].y, 0x07060302u);
        }
    };

    // One K-step s.  At its barrier X(s) and slice(s+1) -- both issued at
    // step s-2 -- must have landed; every step issues the same 3 direct
    // loads (past the end they repeat the last step into a free buffer), so
    // that holds once at most 3 later loads are pending.  (__syncthreads
    // would wait for all of them: its fence counts direct LDS loads as
    // stores.)  The barrier also retires step s-1's reads of the buffers
    // that step s+2 / s+3 now overwrite.
    auto step = [&](uint32_t s, bf16x8 (&bc)[4], bf16x8 (&bn)[4]) {
        asm volatile("s_waitcnt vmcnt(3) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue(clampstep(s + 2), clampstep(s + 3));
        gather(clampstep(s + 1), bn);
        const unsigned char* xs = xbuf + (s % kRing) * kXStepBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bf16x8 af = *reinterpret_cast<const bf16x8*>(xs + (size_t(h) * 128 + i * 32 + n) * 32 + kh * 16);
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bc[f], acc[i][f], 0, 0, 0);
        }
    };

    bf16x8 bA[4], bB[4];
    gather(0, bA);
    uint32_t s = 0;
    for (; s + 1 < nsteps; s += 2) {
        step(s, bA, bB);
        step(s + 1, bB, bA);
    }
    if (s < nsteps) step(s, bA, bB);

    // ---- epilogue: D[m][n] with m = 8*(v/4) + 4*(lane/32) + v%4, n = lane%32
    const int64_t trow = t0 + h * 128 + 4 * kh;      // token of m = 0 in this lane
    const int64_t ocol = o0 + g * 128 + n;           // output of fragment 0
    float* ybase = a.Y + trow * a.M + ocol;
    if (!ok) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[i][f] = float16v{} + __builtin_nanf("");
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int m = i * 32 + 8 * (v >> 2) + (v & 3);
            if (trow + m < a.T) {
#pragma unroll
                for (int f = 0; f < 4; ++f)
                    if (ocol + f * 32 < a.M) __builtin_nontemporal_store(acc[i][f][v], ybase + m * a.M + f * 32);
            }
        }
}

inline size_t tile_lds(const Shape& s) {
    return kRing * kXStepBytes + 4 * idx_ring_bytes(uint32_t(s.R)) + size_t(kO2 / s.R) * s.Bg * 2;
}

inline bool tile_supported(const Shape& s) {
    const bool pow2R = s.R > 0 && (s.R & (s.R - 1)) == 0;
    return pow2R && s.R <= 32 && s.N % kKS == 0 && s.Bg % 8 == 0 && tile_lds(s) <= 160 * 1024;
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
        b.tiles_o = uint32_t((s.M + kO2 - 1) / kO2);
        const int64_t tiles_t = (batch + kT2 - 1) / kT2;
        const int64_t grid = int64_t(b.tiles_o) * tiles_t;
        if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
        gemm_tile_kernel<<<unsigned(grid), 256, tile_lds(s), st>>>(b);
        return launch_status();
    }
    a.tiles_m = uint32_t((s.M + kBN - 1) / kBN);
    const int64_t tiles_t = (batch + kBM - 1) / kBM;
    const int64_t grid = int64_t(a.tiles_m) * tiles_t;
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    gemm_mfma_kernel<<<unsigned(grid), kThreads, lds_bytes(s), st>>>(a);
    return launch_status();
}

}  // namespace sketch

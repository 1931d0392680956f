// gemv.hip -- decode-batch product Y = X * W_hat^T without materialising W_hat.
//
// "Resumen Técnico" › Metodología §4: W_hat = S * P^T.  Because P is one-hot
// and the same for every row block, the product factorises
//     Y[t][b*R + r] = sum_k S[b][k] * Z[t][r][k],   Z[t][r][k] = sum_{j: k(r*N+j)=k} X[t][j]
// (Resultados › Ablación: the matrix form equals the sequential one).
// Z = P^T x costs R*N adds per token and is independent of M; the product
// with S then reads every bucket table exactly once from HBM.
//
// gemv_mfma_kernel (R a power of two <= 16, Bg a multiple of 32):
//   * A workgroup owns RW of the R rows of every block (the "row group") and
//     a set of 16-block tiles.  Small problems split the rows over several
//     workgroups so the chip fills up without any cross-workgroup reduction
//     (every output is written by exactly one workgroup).
//   * It obtains its rows of Z -- computed in place from x through the
//     projection's inverse map (ascending j: deterministic) while that is
//     at most one 4096-column row per workgroup, otherwise (large problems,
//     several tokens) read from the workspace where gemv_z_kernel put it --
//     scales it by a power of two per token (max |Z| -> [2^14, 2^15)) and
//     splits it into binary16 hi + lo parts in LDS.
//   * Matrix cores compute S * Z^T: A = 16 bucket-table rows (binary16,
//     exact), B = hi and lo columns, so every product is exact and the
//     accumulation is float32.  The 4 waves split the K-steps; their partial
//     results are summed in LDS, hi + lo are combined and the scale undone.
//   * If a token's Z is not finite (NaN/Inf in x) or cannot be scaled into
//     binary16 range, the workgroup computes in float32 instead.
// gemv_generic_kernel: float32 fallback for every other shape, after
// gemv_z_kernel has written Z to the workspace.
#include "common.h"

namespace sketch {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;             // 4 waves
constexpr size_t kLdsBudget = 128 * 1024;
constexpr int kMaxTok = 16;               // tokens per launch
constexpr uint32_t kMaxTokInPlace = 4;    // tokens per workgroup when Z is summed in place
constexpr uint64_t kInPlaceZMax = 4096;    // column gathers per workgroup when Z is summed in place, at most
constexpr int kTileBlocks = 16;           // MFMA rows
constexpr int kZThreads = 256;
constexpr size_t kStaticLds = 5 * 1024;   // gemv_mfma_kernel's own shared arrays, at most

__device__ inline bool header_ok(const ProjHeader* h, uint32_t R, uint32_t N, uint32_t Bg, uint32_t seed) {
    return h->magic == kProjMagic && h->version == kProjVersion && h->R == R && h->N == N && h->Bg == Bg &&
           h->seed == seed;
}

// Z of one CSR segment: sum of x over the segment's columns in ascending j.
// Column and x loads go out 8 at a time with clamped indices (no per-element
// branches); entries past the end are masked out of the sum.
template <int XDT>
__device__ inline float segment_sum(const void* X, int64_t xrow, const uint16_t* cols, uint32_t b, uint32_t en) {
    float z = 0.0f;
    for (uint32_t c = b; c < en; c += 8) {
        uint32_t j[8];
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) j[u] = cols[(c + u < en) ? c + u : en - 1];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = load_elem<XDT>(X, xrow + j[u]);
#pragma unroll
        for (int u = 0; u < 8; ++u) z += (c + u < en) ? v[u] : 0.0f;
    }
    return z;
}

// ---------------------------------------------------------------------------
// Z for every (token, row, bucket) into the workspace, plus max |Z| of each
// group of 256 consecutive segments (+Inf when any entry is not finite).
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(kZThreads) void gemv_z_kernel(const void* X, const ProjHeader* hdr, const uint32_t* off,
                                                         const uint16_t* cols, float* Z, float* zmax, int64_t N,
                                                         uint32_t R, uint32_t Bg, uint32_t seed, int64_t t0,
                                                         uint32_t nzc) {
    __shared__ float red[kZThreads / 64];
    const int64_t RB = int64_t(R) * Bg;
    const int64_t t = blockIdx.y;
    const int64_t seg = int64_t(blockIdx.x) * kZThreads + threadIdx.x;
    float z = 0.0f;
    if (seg < RB) {
        if (header_ok(hdr, R, uint32_t(N), Bg, seed))
            z = segment_sum<XDT>(X, (t0 + t) * N, cols, off[seg], off[seg + 1]);
        else
            z = __builtin_nanf("");
        Z[t * RB + seg] = z;
    }
    float m = __builtin_fabsf(z);
    if (!(m <= 3.402823466e38f)) m = __builtin_inff();
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) zmax[t * nzc + blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Element e of an x row in LDS as raw bits (zero-extended binary16 /
// bfloat16 bits, or binary32 bits), and those bits as a float.
template <int XDT>
__device__ inline uint32_t lds_x_bits(const unsigned char* x, uint32_t e) {
    if constexpr (XDT == SKETCH_F32)
        return reinterpret_cast<const uint32_t*>(x)[e];
    else
        return reinterpret_cast<const uint16_t*>(x)[e];
}

template <int XDT>
__device__ inline float x_from_bits(uint32_t v) {
    if constexpr (XDT == SKETCH_F32) {
        return __uint_as_float(v);
    } else if constexpr (XDT == SKETCH_BF16) {
        return bf16_bits_to_f32(uint16_t(v));
    } else {
        return f16_bits_to_f32(uint16_t(v));
    }
}

template <int XDT>
__device__ inline float lds_x(const unsigned char* x, uint32_t e) {
    if constexpr (XDT == SKETCH_F32) {
        return reinterpret_cast<const float*>(x)[e];
    } else if constexpr (XDT == SKETCH_BF16) {
        return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[e]);
    } else {
        return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(x)[e]);
    }
}

// e / Bg without a division sequence: the multiply-high by ceil(2^32 / Bg)
// is the quotient or one more (its error e * (ceil - 2^32/Bg) / 2^32 is
// below 1 for every 32-bit e), and one compare corrects it.
__device__ inline uint32_t div_bg(uint32_t e, uint32_t Bg, uint32_t recip) {
    const uint32_t q = __umulhi(e, recip);
    return q * Bg > e ? q - 1 : q;
}

struct MfmaArgs {
    const uint16_t* S;
    const void* X;
    const ProjHeader* hdr;
    const uint32_t* off;
    const uint16_t* cols;
    const float* Zg;      // global mode: Z from the workspace, [ntok][R][Bg]
    const float* zmaxg;   // global mode: maxima, [ntok][nzc]
    float* Y;
    int64_t nb, M, N, t0;
    uint32_t R, RW, rsplit, Bg, ntok, ntiles, nzc, seed;
    uint32_t tg, tgroups;                  // tokens per workgroup, token groups per tile
    uint32_t bg_recip;                     // ceil(2^32 / Bg), for div_bg
    uint32_t lds_zf, lds_off, lds_cols, lds_x;   // in-place mode: byte offsets of LDS areas
    uint32_t stage_in_frag;                // in-place mode: the staged slices share the fragment area
};

// Copy the bytes [src, src + nbytes) of global memory into LDS at dst with
// direct global->LDS loads (16 bytes per lane), all issued without waiting.
// The copy covers the 16-byte-aligned chunks that hold the range, so it may
// read up to 15 bytes on either side -- never outside the chunks (and pages)
// that hold valid bytes.  Lanes past the last chunk repeat it, so dst must
// have room for roundup(chunks, 64) * 16 bytes.  Returns the offset of src
// inside the first chunk.
__device__ inline uint32_t stage_to_lds(unsigned char* dst, const void* src, uint32_t nbytes, int wave, int lane) {
    const uintptr_t s = reinterpret_cast<uintptr_t>(src);
    const uintptr_t a0 = s & ~uintptr_t(15);
    const uint32_t n = nbytes ? uint32_t((s + nbytes + 15 - a0) >> 4) : 0u;
    for (uint32_t i = uint32_t(wave) * 64; i < n; i += kThreads) {
        const uint32_t c = i + lane < n ? i + lane : n - 1;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(a0 + size_t(c) * 16), dst + size_t(i) * 16, 16,
                                         0, 0);
    }
    return uint32_t(s - a0);
}

constexpr int kPre = 8;   // K-steps per wave of the next tile kept in flight

// MFMAs over the prefetched K-steps wave + 4u (u < kPre); with NEXT each
// register is refilled with the same step of the next tile (nsrow) as soon as
// it has been consumed.
template <int CT, bool NEXT>
__device__ inline void mfma_prefetched(half8 (&pre)[kPre], float4v (&acc)[CT], const half8* frag, int lane, int wave,
                                       uint32_t nst, const uint16_t* nsrow) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
        const uint32_t st = uint32_t(wave) + 4 * u;
        if (st < nst) {
#pragma unroll
            for (int c = 0; c < CT; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pre[u], frag[(st * CT + c) * 64 + lane], acc[c], 0, 0, 0);
        }
        if constexpr (NEXT)
            pre[u] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(nsrow + (st < nst ? st : nst - 1) * 32));
    }
}

// Workgroup barrier that orders LDS accesses only: outstanding global loads
// stay in flight (the fence of __syncthreads would wait for all of them).
__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }


constexpr uint32_t kChunkBytes = 16 * 512;             // 16 bucket-table rows x 256 buckets

// Streaming loop (large stacks, Z from the workspace, all R rows per
// workgroup): every wave owns whole 16-block tiles (wave w of the grid takes
// tiles w, w + 4*grid, ...) and walks all their K-steps itself, so there is
// no cross-wave reduction and no barrier.  A tile streams in chunks of 256
// buckets (8 K-steps): 16 rows x 512 contiguous bytes, loaded as 8
// instructions of 1 KiB (two rows each, 16 bytes per lane) into registers
// one chunk ahead, then written to the wave's LDS slot and read back in the
// MFMA A-fragment pattern (row n = lane % 16); the B fragments (Z hi/lo)
// come from `frag`.  Whole 512-byte row segments per instruction instead of
// 64 bytes of 16 rows is what lets the stream approach the HBM rate
// (measured on this part: 6.7 TB/s for the bare copy pattern, 5.8 TB/s for
// the 16-row one; the same pattern with direct global->LDS loads: 5.8 TB/s).
// The product is computed transposed (Z fragments as A, the tables as B) with
// hi and lo columns interleaved, so after a tile's last chunk every lane adds
// its two (hi, lo) pairs in registers and stores two adjacent outputs.
// Chunk j (of nchunks) of grid wave gw into registers: 8 loads of 1 KiB,
// two 512-byte row segments each (past the end: the last chunk again).
__device__ inline void stream_load_chunk(const MfmaArgs& a, uint32_t gw, uint32_t nwaves, uint32_t nb8,
                                         uint32_t nchunks, uint32_t j, int lane, u32x4v (&v)[8]) {
    const uint32_t jj = j < nchunks ? j : nchunks - 1;
    const uint32_t tile = gw + (jj / nb8) * nwaves, c = jj % nb8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int64_t row = int64_t(tile) * kTileBlocks + 2 * i + (uint32_t(lane) >> 5);
        row = row < a.nb ? row : a.nb - 1;
        v[i] = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4v*>(a.S + row * int64_t(a.Bg) + c * 256 + (uint32_t(lane) & 31) * 8));
    }
}

// `va` holds chunk 0 already (requested before the workgroup's setup).
template <int CT>
__device__ inline void stream_tiles(const MfmaArgs& a, const half8* frag, unsigned char* slots, const float* scale_dn,
                                    int lane, int wave, uint32_t nst, u32x4v (&va)[8]) {
    const uint32_t nwaves = gridDim.x * (kThreads / 64);
    const uint32_t gw = blockIdx.x * (kThreads / 64) + uint32_t(wave);
    if (gw >= a.ntiles) return;
    const uint32_t nb8 = nst / 8;                      // chunks per tile
    const uint32_t my_tiles = (a.ntiles - gw + nwaves - 1) / nwaves;
    const uint32_t nchunks = my_tiles * nb8;
    const uint32_t RW = a.RW, n = uint32_t(lane) & 15u, qd = uint32_t(lane) >> 4;
    unsigned char* ws = slots + size_t(wave) * kChunkBytes;

    auto load_chunk = [&](uint32_t j, u32x4v (&v)[8]) { stream_load_chunk(a, gw, nwaves, nb8, nchunks, j, lane, v); };
    // Transposed product: A = Z hi/lo fragments (16 columns, interleaved
    // layout), B = the 16 bucket-table rows, so D^T[col][block].  Lane
    // (n = lane % 16, qd = lane / 16) holds columns 4qd..4qd+3 of block n:
    // two (hi, lo) pairs of adjacent rows of one token.
    float4v acc[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
    auto finish_tile = [&](uint32_t j) {
        const uint32_t tile = gw + (j / nb8) * nwaves;
        const int64_t blk = int64_t(tile) * kTileBlocks + n;
        if (blk < a.nb) {
#pragma unroll
            for (int c = 0; c < CT; ++c) {
                const uint32_t col0 = uint32_t(c) * 16 + 4 * qd;           // columns col0 .. col0+3
                const uint32_t tt0 = col0 / (2 * RW), rr0 = (col0 % (2 * RW)) / 2;
                const uint32_t tt1 = (col0 + 2) / (2 * RW), rr1 = ((col0 + 2) % (2 * RW)) / 2;
                const float y0 = acc[c][0] + acc[c][1], y1 = acc[c][2] + acc[c][3];
                if (tt0 == tt1 && tt0 < a.ntok) {
                    // rows rr0, rr0 + 1 of one token: 8 contiguous bytes (rr0 even, R
                    // even); non-temporal, as Y is written once (96.5 vs 98.0 us mean
                    // over 4 alternating runs of the 512-table stream)
                    const float2v o = {y0 * scale_dn[tt0], y1 * scale_dn[tt0]};
                    __builtin_nontemporal_store(o, reinterpret_cast<float2v*>(a.Y + (a.t0 + tt0) * a.M + blk * a.R + rr0));
                } else {
                    if (tt0 < a.ntok) a.Y[(a.t0 + tt0) * a.M + blk * a.R + rr0] = y0 * scale_dn[tt0];
                    if (tt1 < a.ntok) a.Y[(a.t0 + tt1) * a.M + blk * a.R + rr1] = y1 * scale_dn[tt1];
                }
            }
        }
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
    };

    u32x4v vb[8];
    auto do_chunk = [&](uint32_t j, const u32x4v (&v)[8]) {
        // rows 2i and 2i+1 of the chunk: lanes 0-31 and 32-63, 512 bytes each
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4v*>(ws + i * 1024 + uint32_t(lane) * 16) = v[i];
        const unsigned char* sl = ws + n * 512 + qd * 16;
        const uint32_t st0 = (j % nb8) * 8;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
            const half8 av = *reinterpret_cast<const half8*>(sl + s8 * 64);
#pragma unroll
            for (int c = 0; c < CT; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(frag[((st0 + s8) * CT + c) * 64 + lane], av, acc[c], 0,
                                                                0, 0);
        }
        if ((j + 1) % nb8 == 0) finish_tile(j);
    };
    for (uint32_t j = 0; j < nchunks; j += 2) {
        load_chunk(j + 1, vb);
        do_chunk(j, va);
        if (j + 1 < nchunks) {
            load_chunk(j + 2, va);
            do_chunk(j + 1, vb);
        }
    }
}

// Column layout of the B operand, per token tt of the workgroup: 2*RW
// columns, hi parts of the group's rows rr = 0..RW-1 first, then the lo
// parts; column c of token tt is MFMA column (tt*2*RW + c) % 16 of column
// tile (tt*2*RW + c) / 16.
//
// ZIN (in-place mode): the workgroup stages its rows' slice of the projection
// (offsets and columns of rows r0..r0+RW-1, which are the CSR positions
// [r0*N, (r0+RW)*N)) and its tokens' x rows into LDS, and sums Z there.
// Otherwise Z comes from the workspace.
template <int XDT, int CT, bool ZIN, bool STREAM>
__global__ __launch_bounds__(kThreads) void gemv_mfma_kernel(MfmaArgs a) {
    static_assert(!(ZIN && STREAM), "the streaming loop takes Z from the workspace");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ uint32_t zmax_bits[kMaxTok];                 // max |Z| of each token (float bits)
    __shared__ uint32_t part_max[ZIN ? kMaxTokInPlace : 1][kThreads];
    __shared__ float scale_up[kMaxTok], scale_dn[kMaxTok];
    __shared__ int tok_fallback[kMaxTok];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    // Workgroups are dealt to the 8 XCDs round robin; renumber them so that
    // the workgroups of one tile (its row and token groups) share an XCD
    // and its L2.
    uint32_t bid = blockIdx.x;
    if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
    const uint32_t per_tile = a.rsplit * a.tgroups;
    const uint32_t rgi = bid % a.rsplit;
    const uint32_t tgi = (bid / a.rsplit) % a.tgroups;
    const uint32_t groups = gridDim.x / per_tile;
    uint32_t tile = bid / per_tile;
    const uint32_t r0 = rgi * a.RW;
    const uint32_t tt0 = tgi * a.tg;
    const uint32_t ntw = a.ntok - tt0 < a.tg ? a.ntok - tt0 : a.tg;   // tokens of this workgroup
    const uint32_t nst = a.Bg / 32;
    const uint32_t nz = ntw * a.RW * a.Bg;                              // Z values of this workgroup

    half8* frag = reinterpret_cast<half8*>(lds);                                        // [nst][CT][64]
    float4v* red = reinterpret_cast<float4v*>(lds + size_t(nst) * CT * 64 * 16);        // [4][CT][64]
    float* zf = reinterpret_cast<float*>(lds + a.lds_zf);   // in-place: [ntw][RW][Bg] float32

    // ---- loads that do not depend on Z go out first: the projection header,
    // the staged slices (in-place mode), then the first tile's bucket rows
    const uint4v h0 = reinterpret_cast<const uint4v*>(a.hdr)[0];   // magic, version, R, N
    const uint4v h1 = reinterpret_cast<const uint4v*>(a.hdr)[1];   // Bg, seed, padding
    __builtin_amdgcn_sched_barrier(0);
    uint32_t sh_off = 0, sh_cols = 0, sh_x = 0;
    if constexpr (ZIN) {
        const uint32_t xb = XDT == SKETCH_F32 ? 4u : 2u;
        sh_off = stage_to_lds(lds + a.lds_off, a.off + size_t(r0) * a.Bg, (a.RW * a.Bg + 1) * 4u, wave, lane);
        sh_cols = stage_to_lds(lds + a.lds_cols, a.cols + size_t(r0) * a.N, a.RW * uint32_t(a.N) * 2u, wave, lane);
        sh_x = stage_to_lds(lds + a.lds_x,
                            static_cast<const unsigned char*>(a.X) + size_t(a.t0 + tt0) * size_t(a.N) * xb,
                            ntw * uint32_t(a.N) * xb, wave, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
    half8 pre[kPre];
    {
        int64_t row0 = int64_t(tile) * kTileBlocks + (lane & 15);
        row0 = row0 < a.nb ? row0 : a.nb - 1;            // rows past the end are loaded but never stored
        const uint16_t* srow = a.S + row0 * int64_t(a.Bg) + (lane >> 4) * 8;
#pragma unroll
        for (int u = 0; u < kPre; ++u) {
            const uint32_t st = wave + 4 * u < nst ? wave + 4 * u : nst - 1;
            pre[u] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(srow + st * 32));
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    const bool ok = h0.x == kProjMagic && h0.y == kProjVersion && h0.z == a.R && h0.w == uint32_t(a.N) &&
                    h1.x == a.Bg && h1.y == a.seed;
    if (tid < kMaxTok) zmax_bits[tid] = 0;
    if constexpr (ZIN) {
        if (!a.stage_in_frag)
            for (uint32_t f = tid; f < nst * CT * 64; f += kThreads) frag[f] = half8{};
    }

    // ---- streaming: this wave's first chunk of bucket rows goes out before
    // the setup below and lands while it runs
    u32x4v sva[8];
    if constexpr (STREAM) {
        const uint32_t nwaves = gridDim.x * (kThreads / 64), gw = blockIdx.x * (kThreads / 64) + uint32_t(wave);
        if (gw < a.ntiles) {
            const uint32_t my_tiles = (a.ntiles - gw + nwaves - 1) / nwaves;
            stream_load_chunk(a, gw, nwaves, nst / 8, my_tiles * (nst / 8), 0, lane, sva);
        }
    }

    // ---- Z from the workspace (not in place): the first round of fragment
    // loads goes out now, with the maxima below, so both take one trip
    const uint32_t lgRW = __builtin_ctz(a.RW);   // RW is a power of two
    const uint32_t nfrag = nst * CT * 64;
    constexpr int FB = 8;                        // fragments per thread and round (16 loads in flight)
    // fragment f = 8 buckets of one (token, row, hi|lo) column -- layout below
    auto frag_load = [&](uint32_t f, float4v (&zv)[2], uint32_t& tt, uint32_t& h) {
        f = f < nfrag ? f : nfrag - 1;
        const uint32_t c16 = f & 15, kq = (f >> 4) & 3, sct = f >> 6;
        const uint32_t ct = sct % CT, st = sct / CT;
        const uint32_t col = ct * 16 + c16, w = col & (2 * a.RW - 1);
        tt = col >> (lgRW + 1);
        uint32_t rr;
        if constexpr (STREAM) {
            rr = w >> 1;
            h = w & 1;
        } else {
            rr = w & (a.RW - 1);
            h = w >> lgRW;
        }
        const uint32_t ttc = tt < ntw ? tt : 0;
        const float* zp = a.Zg + (size_t(tt0 + ttc) * a.R + r0 + rr) * a.Bg + st * 32 + kq * 8;
        zv[0] = *reinterpret_cast<const float4v*>(zp);
        zv[1] = *reinterpret_cast<const float4v*>(zp + 4);
    };
    auto frag_store = [&](uint32_t f, const float4v (&zv)[2], uint32_t tt, uint32_t h) {
        half8 out = half8{};
        if (tt < ntw) {
            const float sc = scale_up[tt];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = zv[e >> 2][e & 3] * sc;
                const _Float16 hi = static_cast<_Float16>(v);
                out[e] = h ? static_cast<_Float16>(v - static_cast<float>(hi)) : hi;
            }
        }
        frag[f] = out;
    };
    float4v zv0[FB][2];
    uint32_t ztt0[FB], zh0[FB];
    if constexpr (!ZIN) {
#pragma unroll
        for (int u = 0; u < FB; ++u) frag_load(tid + u * kThreads, zv0[u], ztt0[u], zh0[u]);
    }

    // ---- token maxima of |Z|
    if constexpr (!ZIN) {
        for (uint32_t i = tid; i < ntw * a.nzc; i += kThreads) {
            const float m = a.zmaxg[size_t(tt0) * a.nzc + i];
            atomicMax(&zmax_bits[i / a.nzc], (m <= 3.402823466e38f) ? __float_as_uint(m) : 0x7F800000u);
        }
    } else {
        // the header and the staged slices have landed once only the kPre
        // bucket-row loads are left
        // (__syncthreads would also wait for those: its fence counts the
        // direct-to-LDS loads as stores and drains every outstanding load)
        static_assert(kPre == 8, "the wait below counts the bucket-row loads");
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        const uint32_t* offl = reinterpret_cast<const uint32_t*>(lds + a.lds_off + sh_off);
        const uint16_t* coll = reinterpret_cast<const uint16_t*>(lds + a.lds_cols + sh_cols);
        const unsigned char* xl = lds + a.lds_x + sh_x;
        const uint32_t base = r0 * uint32_t(a.N), npos = a.RW * uint32_t(a.N), N32 = uint32_t(a.N);
        // entry e = (tt * RW + rr) * Bg + k, 4 per thread at a time; every
        // LDS read is unconditional (indices clamped, dead entries masked)
        constexpr int U = 4;
        uint32_t mx[kMaxTokInPlace] = {};   // this thread's max |Z| bits per token
        for (uint32_t e0 = tid; e0 < nz; e0 += U * kThreads) {
            uint32_t b[U], en[U], xo[U], tts[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t e = e0 + u * kThreads < nz ? e0 + u * kThreads : nz - 1;
                const uint32_t trr = div_bg(e, a.Bg, a.bg_recip), k = e - trr * a.Bg;
                const uint32_t rr = trr & (a.RW - 1), tt = trr >> lgRW;
                const uint32_t sl = rr * a.Bg + k;
                uint32_t lo = offl[sl] - base, hi = offl[sl + 1] - base;
                hi = hi < npos ? hi : npos;
                lo = lo < hi ? lo : hi;
                b[u] = lo;
                en[u] = hi;
                xo[u] = tt * N32;
                tts[u] = tt;
            }
            // The column reads of all U entries, then all their x reads, go
            // out before any result is used (the scheduling barriers keep
            // the compiler from serialising the entries into one LDS round
            // trip each); x is read as raw bits and widened afterwards.
            uint32_t j[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < 8; ++v) j[u][v] = coll[b[u] + v < npos ? b[u] + v : npos - 1];
            __builtin_amdgcn_sched_barrier(0);
            uint32_t xr[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int v = 0; v < 8; ++v) xr[u][v] = lds_x_bits<XDT>(xl, xo[u] + (j[u][v] < N32 ? j[u][v] : N32 - 1));
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float acc = 0.0f;
#pragma unroll
                for (int v = 0; v < 8; ++v) acc += (b[u] + v < en[u]) ? x_from_bits<XDT>(xr[u][v]) : 0.0f;
                for (uint32_t c = b[u] + 8; c < en[u]; ++c) {
                    const uint32_t jj = coll[c];
                    acc += lds_x<XDT>(xl, xo[u] + (jj < N32 ? jj : N32 - 1));
                }
                const uint32_t e = e0 + u * kThreads;
                if (e < nz) {
                    const float z = ok ? acc : __builtin_nanf("");
                    zf[e] = z;
                    const float m = __builtin_fabsf(z);
                    const uint32_t mb = (m <= 3.402823466e38f) ? __float_as_uint(m) : 0x7F800000u;
#pragma unroll
                    for (uint32_t q = 0; q < kMaxTokInPlace; ++q) mx[q] = (tts[u] == q && mb > mx[q]) ? mb : mx[q];
                }
            }
        }
        // token maxima: plain LDS stores and a wave reduction (an LDS atomic
        // here would make the compiler wait for every outstanding load)
#pragma unroll
        for (uint32_t q = 0; q < kMaxTokInPlace; ++q) part_max[q][tid] = mx[q];
        lds_barrier();
        // every staged slice has been read: when they share the fragment
        // area it is cleared only now (two barriers before the scatter)
        if (a.stage_in_frag)
            for (uint32_t f = tid; f < nst * CT * 64; f += kThreads) frag[f] = half8{};
        if (uint32_t(wave) < ntw) {
            uint32_t m = 0;
#pragma unroll
            for (int i = 0; i < kThreads / 64; ++i) m = part_max[wave][lane + 64 * i] > m ? part_max[wave][lane + 64 * i] : m;
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) {
                const uint32_t t = uint32_t(__shfl_xor(int(m), o));
                m = t > m ? t : m;
            }
            if (lane == 0) zmax_bits[wave] = m;
        }
    }
    if constexpr (ZIN) lds_barrier(); else __syncthreads();
    if (tid < int(ntw)) {
        const float m = __uint_as_float(zmax_bits[tid]);
        int e = 0, f = 0;
        if (!(m <= 3.402823466e38f)) {
            f = 1;
        } else if (m > 0.0f) {
            e = 14 - ilogbf(m);
            if (e > 120 || e < -120) f = 1;
        }
        scale_up[tid] = ldexpf(1.0f, e);
        scale_dn[tid] = ldexpf(1.0f, -e);
        tok_fallback[tid] = f;
    }
    if constexpr (ZIN) lds_barrier(); else __syncthreads();
    // float32 for the whole workgroup if any of its tokens needs it
    bool fb = false;
    for (uint32_t t = 0; t < ntw; ++t) fb = fb || tok_fallback[t] != 0;

    // ---- binary16 hi/lo fragments
    // frag[(s*CT + ct)*64 + kq*16 + c16] = 8 buckets k = 32 s + 8 kq + 0..7 of
    // column ct*16 + c16.  A column is the hi or lo part of (token tt, row rr):
    // split layout  col = tt*2RW + h*RW + rr   (workgroup tile loop),
    // interleaved   col = tt*2RW + 2 rr + h    (streaming loop: the pair sits
    // in one lane of the transposed product).  Columns past the tokens are 0.
    if constexpr (ZIN) {
        // Z in LDS, few columns in use (small batches): the fragments were
        // cleared at kernel start (after the Z sums when the staged slices
        // shared their area); scatter every Z value's hi and lo parts (split
        // layout)
        if (!fb) {
            _Float16* fh = reinterpret_cast<_Float16*>(frag);
            for (uint32_t e = tid; e < nz; e += kThreads) {
                const uint32_t trr = div_bg(e, a.Bg, a.bg_recip), k = e - trr * a.Bg;
                const uint32_t rr = trr & (a.RW - 1), tt = trr >> lgRW;
                const float v = zf[e] * scale_up[tt];
                const _Float16 hi = static_cast<_Float16>(v);
                const _Float16 lo = static_cast<_Float16>(v - static_cast<float>(hi));
                const uint32_t s = k >> 5, w32 = k & 31;
                const uint32_t chi = tt * 2 * a.RW + rr, clo = chi + a.RW;
                fh[size_t((s * CT + (chi >> 4)) * 64 + (w32 >> 3) * 16 + (chi & 15)) * 8 + (w32 & 7)] = hi;
                fh[size_t((s * CT + (clo >> 4)) * 64 + (w32 >> 3) * 16 + (clo & 15)) * 8 + (w32 & 7)] = lo;
            }
        }
    } else if (!fb) {
#pragma unroll
        for (int u = 0; u < FB; ++u)
            if (tid + u * kThreads < nfrag) frag_store(tid + u * kThreads, zv0[u], ztt0[u], zh0[u]);
        for (uint32_t f0 = tid + FB * kThreads; f0 < nfrag; f0 += FB * kThreads) {
            float4v zv[FB][2];
            uint32_t tt_[FB], h_[FB];
#pragma unroll
            for (int u = 0; u < FB; ++u) frag_load(f0 + u * kThreads, zv[u], tt_[u], h_[u]);
#pragma unroll
            for (int u = 0; u < FB; ++u)
                if (f0 + u * kThreads < nfrag) frag_store(f0 + u * kThreads, zv[u], tt_[u], h_[u]);
        }
    }
    if constexpr (ZIN) lds_barrier(); else __syncthreads();

    if constexpr (STREAM) {
        if (!fb) {
            stream_tiles<CT>(a, frag, lds + a.lds_zf, scale_dn, lane, wave, nst, sva);
            return;
        }
    }

    for (; tile < a.ntiles; tile += groups) {
        const int64_t b0 = int64_t(tile) * kTileBlocks;
        if (!fb) {
            int64_t row = b0 + (lane & 15);
            row = row < a.nb ? row : a.nb - 1;
            const uint16_t* srow = a.S + row * int64_t(a.Bg) + (lane >> 4) * 8;
            float4v acc[CT];
#pragma unroll
            for (int c = 0; c < CT; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};
            // steps wave + 4u for u < kPre come from the prefetch; once a step
            // is consumed its register takes the next tile's same step
            const uint32_t nxt = tile + groups;
            if (nxt < a.ntiles) {
                int64_t nrow = int64_t(nxt) * kTileBlocks + (lane & 15);
                nrow = nrow < a.nb ? nrow : a.nb - 1;
                mfma_prefetched<CT, true>(pre, acc, frag, lane, wave, nst, a.S + nrow * int64_t(a.Bg) + (lane >> 4) * 8);
            } else {
                mfma_prefetched<CT, false>(pre, acc, frag, lane, wave, nst, nullptr);
            }
            uint32_t s = wave + 4 * kPre;
            for (; s + 28 < nst; s += 32) {
                half8 av[8];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    av[u] = __builtin_nontemporal_load(reinterpret_cast<const half8*>(srow + (s + 4 * u) * 32));
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int c = 0; c < CT; ++c)
                        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[u], frag[((s + 4 * u) * CT + c) * 64 + lane],
                                                                        acc[c], 0, 0, 0);
            }
            for (; s < nst; s += 4) {
                const half8 av = __builtin_nontemporal_load(reinterpret_cast<const half8*>(srow + s * 32));
#pragma unroll
                for (int c = 0; c < CT; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, frag[(s * CT + c) * 64 + lane], acc[c], 0, 0, 0);
            }
#pragma unroll
            for (int c = 0; c < CT; ++c) red[(wave * CT + c) * 64 + lane] = acc[c];
            __syncthreads();
            // sum the K-slices of the 4 waves; lane holds D[4*(lane/16)+i][lane%16]
            for (int c = wave; c < CT; c += 4) {
                float4v v = red[c * 64 + lane];
#pragma unroll
                for (int w = 1; w < 4; ++w) v += red[(w * CT + c) * 64 + lane];
                red[c * 64 + lane] = v;
            }
            __syncthreads();
            // outputs: (tt, rr, block) -> hi + lo columns, unscaled
            const uint32_t nout = ntw * a.RW * kTileBlocks;
            for (uint32_t o = tid; o < nout; o += kThreads) {
                const uint32_t bi = o % kTileBlocks, trr = o / kTileBlocks;
                const uint32_t rr = trr & (a.RW - 1), tt = trr >> lgRW;
                const int64_t blk = b0 + bi;
                if (blk >= a.nb) continue;
                const uint32_t chi = tt * 2 * a.RW + rr, clo = chi + a.RW;
                const uint32_t li = (bi >> 2) * 16;     // lane group of row bi
                const float hi = red[(chi >> 4) * 64 + li + (chi & 15)][bi & 3];
                const float lo = red[(clo >> 4) * 64 + li + (clo & 15)][bi & 3];
                a.Y[(a.t0 + tt0 + tt) * a.M + blk * a.R + r0 + rr] = (hi + lo) * scale_dn[tt];
            }
        } else {
            // float32: thread per (token, block, row) output of the tile
            const uint32_t nout = ntw * kTileBlocks * a.RW;
            for (uint32_t o = tid; o < nout; o += kThreads) {
                const uint32_t rr = o % a.RW, bi = (o / a.RW) % kTileBlocks, tt = o / (a.RW * kTileBlocks);
                const int64_t blk = b0 + bi;
                if (blk >= a.nb) continue;
                const uint16_t* sb = a.S + blk * int64_t(a.Bg);
                const float* zr;
                if constexpr (ZIN)
                    zr = zf + (size_t(tt) * a.RW + rr) * a.Bg;
                else
                    zr = a.Zg + (size_t(tt0 + tt) * a.R + r0 + rr) * a.Bg;
                float acc = 0.0f;
                for (uint32_t k = 0; k < a.Bg; ++k) acc += f16_bits_to_f32(sb[k]) * zr[k];
                a.Y[(a.t0 + tt0 + tt) * a.M + blk * a.R + r0 + rr] = acc;
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Generic float32 fallback (other shapes): Z from the workspace.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemv_generic_kernel(const uint16_t* S, const float* Z, float* Y,
                                                           int64_t nb, int64_t M, uint32_t R, uint32_t Bg,
                                                           int64_t batch, int64_t t0) {
    __shared__ float red[4];
    const int tid = threadIdx.x;
    const int64_t RB = int64_t(R) * Bg;
    for (int64_t b = blockIdx.x; b < nb; b += gridDim.x) {
        const uint16_t* Sb = S + b * Bg;
        for (int64_t t = 0; t < batch; ++t) {
            for (uint32_t r = 0; r < R; ++r) {
                const float* z = Z + t * RB + int64_t(r) * Bg;
                float acc = 0.0f;
                for (uint32_t k = tid; k < Bg; k += 256) acc += f16_bits_to_f32(Sb[k]) * z[k];
                for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
                if ((tid & 63) == 0) red[tid >> 6] = acc;
                __syncthreads();
                if (tid == 0) Y[(t0 + t) * M + b * R + r] = red[0] + red[1] + red[2] + red[3];
                __syncthreads();
            }
        }
    }
}

int num_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu;
}

// Launch plan for passes of up to ntok_pass tokens.
struct Plan {
    bool mfma, zsrc_global, stream, stage_in_frag;
    uint32_t RW, rsplit, CT, ntok_pass, tg, ntiles, nzc;
    uint32_t lds_zf, lds_off, lds_cols, lds_x;
    size_t lds;
};

// LDS a direct copy of nbytes needs (see stage_to_lds).
inline size_t stage_bytes(size_t nbytes) { return ((nbytes / 16 + 2 + 63) / 64) * 64 * 16; }

inline uint32_t ct_for(uint32_t ntok, uint32_t RW) {
    uint32_t ct = (ntok * 2 * RW + 15) / 16, c2 = 1;
    while (c2 < ct) c2 <<= 1;
    return c2;
}

// LDS layout: fragments | partial sums | (in-place) Z | offsets | columns | x.
// The staged offsets, columns and x are dead once Z is summed, before the
// fragments are built: when they fit the fragment and partial-sum area they
// go there instead of after Z.
inline void set_lds(Plan& p, const Shape& s, uint32_t tg, uint32_t xb) {
    const uint32_t nst = uint32_t(s.Bg / 32);
    p.tg = tg;
    p.CT = ct_for(tg, p.RW);
    const size_t front = size_t(nst) * p.CT * 64 * 16 + size_t(4) * p.CT * 64 * 16;
    size_t at = front;
    p.lds_zf = p.lds_off = p.lds_cols = p.lds_x = uint32_t(at);
    p.stage_in_frag = false;
    if (!p.zsrc_global) {
        p.lds_zf = uint32_t(at);
        at += size_t(tg) * p.RW * s.Bg * 4;
        const size_t so = stage_bytes(size_t(p.RW) * s.Bg * 4 + 4), sc = stage_bytes(size_t(p.RW) * s.N * 2),
                     sx = stage_bytes(size_t(tg) * s.N * xb);
        p.stage_in_frag = so + sc + sx <= front;
        size_t st = p.stage_in_frag ? 0 : at;
        p.lds_off = uint32_t(st);
        p.lds_cols = uint32_t(st + so);
        p.lds_x = uint32_t(st + so + sc);
        st += so + sc + sx;
        at = at > st ? at : st;
    }
    p.lds = at;
}

Plan make_plan(const Shape& s, int64_t batch, sketch_dtype xdt, int ncu) {
    Plan p{};
    const bool pow2R = s.R > 0 && (s.R & (s.R - 1)) == 0;
    const uint32_t xb = xdt == SKETCH_F32 ? 4u : 2u;
    p.mfma = pow2R && s.R <= 16 && s.Bg % 32 == 0;
    p.ntiles = uint32_t((s.nb + kTileBlocks - 1) / kTileBlocks);
    p.nzc = uint32_t((s.R * s.Bg + kZThreads - 1) / kZThreads);
    p.ntok_pass = uint32_t(batch < kMaxTok ? batch : kMaxTok);
    if (p.ntok_pass < 1) p.ntok_pass = 1;
    if (!p.mfma) return p;
    const uint32_t target = uint32_t(2 * ncu);
    // Small problems split the rows (and tokens) over workgroups and compute
    // Z in place; large ones compute Z once in its own kernel and give every
    // workgroup all the rows and tokens of a pass.
    uint32_t rsplit = 1;
    while (rsplit < uint32_t(s.R) && p.ntiles * rsplit < target) rsplit <<= 1;
    p.rsplit = rsplit;
    p.RW = uint32_t(s.R) / rsplit;
    p.zsrc_global = p.ntiles >= target;
    if (!p.zsrc_global) {
        uint32_t tg = p.ntok_pass < kMaxTokInPlace ? p.ntok_pass : kMaxTokInPlace;
        for (;; --tg) {
            set_lds(p, s, tg, xb);
            if (p.lds <= kLdsBudget || tg == 1) break;
        }
        // In place, every tile group recomputes its rows' Z, so each
        // workgroup sums tg * RW * N gathers from LDS; past one 4096-column
        // row per workgroup a single Z pass in its own kernel costs less
        // (4096 x 4096 at 0.5 bpw: 7.6 us in place vs 9.6 at batch 1, 10.4
        // vs 9.9 at batch 2, 36 vs 15 at batch 16).
        if (p.lds > kLdsBudget || uint64_t(p.tg) * p.RW * uint64_t(s.N) > kInPlaceZMax) p.zsrc_global = true;
    }
    if (p.zsrc_global) {
        uint32_t ntok = p.ntok_pass;
        for (;; --ntok) {
            set_lds(p, s, ntok, xb);
            if (p.lds <= kLdsBudget || ntok == 1) break;
        }
        p.ntok_pass = ntok;
        // one token column tile: the wave-streaming loop, its LDS slots
        // replacing the partial-sum area
        const size_t frag_bytes = size_t(s.Bg / 32) * p.CT * 64 * 16;
        const size_t stream_lds = frag_bytes + size_t(kThreads / 64) * kChunkBytes;
        if (p.lds <= kLdsBudget && p.CT == 1 && p.rsplit == 1 && (s.Bg / 32) % 8 == 0 && stream_lds <= kLdsBudget) {
            p.stream = true;
            p.lds_zf = uint32_t(frag_bytes);
            p.lds = stream_lds;
        }
        if (p.lds > kLdsBudget) {
            p.mfma = false;
            p.zsrc_global = false;
            p.ntok_pass = uint32_t(batch < kMaxTok ? batch : kMaxTok);
            if (p.ntok_pass < 1) p.ntok_pass = 1;
        }
    }
    return p;
}

// Workgroups of a pass of ntok tokens: about one round of them (two per CU,
// or one when the LDS of two does not fit a CU's 160 KiB).
inline uint32_t plan_grid(const Plan& p, uint32_t ntok, uint32_t* tgroups, int ncu) {
    *tgroups = (ntok + p.tg - 1) / p.tg;
    const uint32_t per_tile = p.rsplit * *tgroups;
    const uint32_t per_cu = 2 * (p.lds + kStaticLds) <= size_t(160) * 1024 ? 2u : 1u;
    const uint32_t target = per_cu * uint32_t(ncu);
    const uint32_t want = (target + per_tile - 1) / per_tile;
    const uint32_t groups = p.ntiles < want ? p.ntiles : want;
    return groups * per_tile;
}

template <int XDT, int CT>
void launch_mfma(const MfmaArgs& a, const Plan& p, uint32_t grid, hipStream_t st) {
    if (p.stream)
        gemv_mfma_kernel<XDT, CT, false, true><<<grid, kThreads, p.lds, st>>>(a);
    else if (p.zsrc_global)
        gemv_mfma_kernel<XDT, CT, false, false><<<grid, kThreads, p.lds, st>>>(a);
    else
        gemv_mfma_kernel<XDT, CT, true, false><<<grid, kThreads, p.lds, st>>>(a);
}

template <int XDT>
void launch_mfma_ct(const MfmaArgs& a, const Plan& p, uint32_t grid, hipStream_t st) {
    switch (p.CT) {
        case 1: launch_mfma<XDT, 1>(a, p, grid, st); break;
        case 2: launch_mfma<XDT, 2>(a, p, grid, st); break;
        case 4: launch_mfma<XDT, 4>(a, p, grid, st); break;
        case 8: launch_mfma<XDT, 8>(a, p, grid, st); break;
        default: launch_mfma<XDT, 16>(a, p, grid, st); break;
    }
}

template <int XDT>
void launch_z(const void* X, const ProjHeader* hdr, const uint32_t* off, const uint16_t* cols, float* Z, float* zmax,
              const Shape& s, uint32_t seed, int64_t t0, int64_t ntok, uint32_t nzc, hipStream_t st) {
    dim3 g(nzc, unsigned(ntok));
    gemv_z_kernel<XDT><<<g, kZThreads, 0, st>>>(X, hdr, off, cols, Z, zmax, s.N, uint32_t(s.R), uint32_t(s.Bg), seed,
                                                t0, nzc);
}

}  // namespace

// Workspace: [Z: ntok_pass x R x Bg float32][Z maxima: ntok_pass x nzc]; the
// in-place path of small problems needs none.
size_t gemv_workspace_bytes(const Shape& s, int64_t batch, sketch_dtype xdt) {
    const Plan p = make_plan(s, batch, xdt, num_cus());
    if (p.mfma && !p.zsrc_global) return 0;
    return align256(sizeof(float) * size_t(p.ntok_pass) * s.R * s.Bg) +
           align256(sizeof(float) * size_t(p.ntok_pass) * p.nzc);
}

sketch_status launch_gemv(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                          const void* X, sketch_dtype xdt, int64_t batch, float* Y, void* ws, hipStream_t st) {
    const ProjLayout L = proj_layout(s.R, s.N, s.Bg);
    const char* pb = static_cast<const char*>(proj);
    const auto* hdr = reinterpret_cast<const ProjHeader*>(pb);
    const auto* off = reinterpret_cast<const uint32_t*>(pb + L.off);
    const auto* cols = reinterpret_cast<const uint16_t*>(pb + L.cols);
    const int ncu = num_cus();
    const Plan plan = make_plan(s, batch, xdt, ncu);
    const bool need_z = !plan.mfma || plan.zsrc_global;
    float* Z = static_cast<float*>(ws);
    float* zmax = need_z ? reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                    align256(sizeof(float) * size_t(plan.ntok_pass) * s.R * s.Bg))
                         : nullptr;

    for (int64_t t0 = 0; t0 < batch; t0 += plan.ntok_pass) {
        const int64_t ntok = batch - t0 < int64_t(plan.ntok_pass) ? batch - t0 : int64_t(plan.ntok_pass);
        if (need_z) {
            switch (xdt) {
                case SKETCH_F32: launch_z<SKETCH_F32>(X, hdr, off, cols, Z, zmax, s, p->seed, t0, ntok, plan.nzc, st); break;
                case SKETCH_BF16: launch_z<SKETCH_BF16>(X, hdr, off, cols, Z, zmax, s, p->seed, t0, ntok, plan.nzc, st); break;
                case SKETCH_F16: launch_z<SKETCH_F16>(X, hdr, off, cols, Z, zmax, s, p->seed, t0, ntok, plan.nzc, st); break;
            }
            if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
        }
        if (!plan.mfma) {
            const int grid = int(s.nb < 4096 ? s.nb : 4096);
            gemv_generic_kernel<<<grid, 256, 0, st>>>(tables, Z, Y, s.nb, s.M, uint32_t(s.R), uint32_t(s.Bg), ntok,
                                                      t0);
        } else {
            MfmaArgs a;
            a.S = tables;
            a.X = X;
            a.hdr = hdr;
            a.off = off;
            a.cols = cols;
            a.Zg = Z;
            a.zmaxg = zmax;
            a.Y = Y;
            a.nb = s.nb;
            a.M = s.M;
            a.N = s.N;
            a.t0 = t0;
            a.R = uint32_t(s.R);
            a.RW = plan.RW;
            a.rsplit = plan.rsplit;
            a.Bg = uint32_t(s.Bg);
            a.seed = p->seed;
            a.ntok = uint32_t(ntok);
            a.ntiles = plan.ntiles;
            a.nzc = plan.nzc;
            a.tg = plan.tg;
            a.bg_recip = uint32_t(((uint64_t(1) << 32) + uint64_t(s.Bg) - 1) / uint64_t(s.Bg));
            const uint32_t grid = plan_grid(plan, uint32_t(ntok), &a.tgroups, ncu);
            a.lds_zf = plan.lds_zf;
            a.lds_off = plan.lds_off;
            a.lds_cols = plan.lds_cols;
            a.lds_x = plan.lds_x;
            a.stage_in_frag = plan.stage_in_frag ? 1u : 0u;
            switch (xdt) {
                case SKETCH_F32: launch_mfma_ct<SKETCH_F32>(a, plan, grid, st); break;
                case SKETCH_BF16: launch_mfma_ct<SKETCH_BF16>(a, plan, grid, st); break;
                case SKETCH_F16: launch_mfma_ct<SKETCH_F16>(a, plan, grid, st); break;
            }
        }
        if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    }
    return SKETCH_OK;
}

}  // namespace sketch

// dgemm.h -- prefill product Y = X * W_hat^T with W_hat decoded weight by
// weight into LDS, 32 columns at a time: the one kernel skeleton of the
// sketch variants whose weights the tile kernel (gemm.hip) cannot gather
// as table words shared by all fragments of a lane -- the multi-row sketch
// (a pick among the rows' candidates, "Resumen Técnico" › Metodología §1),
// the importance-aware allocation (a bucket count of its own per block,
// Metodología §2) -- and of the 4-bit sketch (Resultados) on the shapes the
// tile kernel does not take.  Decompression as a matrix product:
// Metodología §4.
//
// Tile: 64 tokens per wave (D::kThreads / 64 waves) x 128 outputs; every
// wave owns all 128 outputs (2 x 4 MFMA 32x32x16 bf16, fp32 accumulate),
// so one decoded weight feeds every token of the tile.
//   * The tables of the tile's row blocks are staged in LDS once (D).
//   * K runs in 32-column chunks.  For chunk c the MFMAs read W_hat[c] from
//     LDS and X[c] from registers; meanwhile the workgroup decodes chunk c+1
//     into the other W_hat buffer (D decodes D::kCols weights of one output
//     row per thread), X[c+1] is loaded into registers, the map slices of
//     chunk c+3 (the 16-byte pieces of index or hash maps a chunk needs,
//     one per thread at most) are loaded into registers and those of chunk
//     c+2, loaded one chunk earlier, are stored to LDS.  Every wait is thus
//     for loads issued a whole chunk before; one barrier per chunk.
//   * Loads go out unconditionally from clamped, in-bounds addresses and the
//     loop is unrolled by two over alternating register sets, so the wait
//     counters see the same loads on every path and no result is copied.
//   * k order inside a chunk: lane (m, h) of an A fragment holds, at MFMA
//     step ks, columns 16h + 8ks .. 16h + 8ks + 7 of its token, so a lane
//     reads its 32 contiguous bytes of X with two 16-byte loads; B fragments
//     read W_hat at the same columns (the sum over k is the same).
//
// A decode policy D provides:
//   Args                         kernel arguments with X (bf16 bits), Y, T, M, N
//   kThreads, kSchedLds, kSchedValu   workgroup size; LDS reads and VALU
//                                instructions to place after each MFMA
//   kScaled                      outputs carry a per-output factor
//   D(args, region, tid, o0, o_d, jseg)   per-thread state; region: its LDS
//                                after the two W_hat buffers
//   header_ok()                  the projection matches (uniform)
//   stage()                      the tables of the tile's blocks into LDS
//   map_load(j0, v), map_store(buf, v)   the thread's map slice of chunk j0
//   decode(buf, j0, dst)         bfloat16 weights of output row o_d, chunk
//                                columns jseg .. jseg + kCols - 1 (0 past N)
//                                from map buffer buf, into dst
//   out_scale(col)               the per-output factor (kScaled only)
//
// K split: when the tiles would leave CUs idle (the multi-row sketch's
// 512-token tiles: 128 of them for 2048 tokens x 4096 outputs), ksplit
// workgroups share a tile, each taking an even run of its K-chunks; part 0
// writes Y, part h > 0 its own float32 buffer, and dgemm_add_kernel adds the
// parts to Y in part order (the same bits on every call).
#pragma once
#include "common.h"

namespace sketch {
namespace dgemm {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kTN = 128;         // outputs per tile
constexpr int kBK = 32;          // columns per K-chunk
constexpr int kLd = kBK + 8;     // W_hat LDS row stride (elements)

// Bytes of LDS before a policy's region (two W_hat buffers).
constexpr size_t kWBytes = size_t(2) * kTN * kLd * 2;

// Weights of one chunk a thread decodes.
template <int THREADS>
constexpr int cols_per_thread() { return kTN * kBK / THREADS; }

template <class D>
__global__ __launch_bounds__(D::kThreads, 1) void dgemm_kernel(typename D::Args a, uint32_t tiles_m, uint32_t ksplit,
                                                               float* part) {
    constexpr int kThreads = D::kThreads;
    constexpr int kTM = kThreads;                       // tokens per tile: 64 per wave
    constexpr int kCols = cols_per_thread<kThreads>();
    static_assert(kCols == 8 || kCols == 16, "a thread decodes 8 or 16 columns of one row");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    uint16_t* Ws = reinterpret_cast<uint16_t*>(lds_raw);   // [2][kTN][kLd]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // workgroup = (part h, tile); part h > 0 writes part[(h - 1) * T * M ...]
    const uint32_t ntile = tiles_m * uint32_t((a.T + kTM - 1) / kTM);
    const uint32_t h = blockIdx.x / ntile, tix = blockIdx.x % ntile;
    const int64_t tile_m = tix % tiles_m, tile_t = tix / tiles_m;
    const int64_t o0 = tile_m * kTN, t0 = tile_t * kTM;
    const uint16_t* X = static_cast<const uint16_t*>(a.X);
    // decode assignment: output row o_d of the tile, chunk columns jseg .. jseg + kCols - 1
    const int o_d = tid / (kBK / kCols), jseg = (tid % (kBK / kCols)) * kCols;
    D d(a, lds_raw + kWBytes, tid, o0, o_d, jseg);

    if (!d.header_ok()) {   // uniform: NaN tile, nothing else read
        for (int u = tid; u < kTM * kTN; u += kThreads) {
            const int64_t t = t0 + u / kTN, o = o0 + u % kTN;
            if (t < a.T && o < a.M) a.Y[t * a.M + o] = __builtin_nanf("");
        }
        return;
    }
    d.stage();

    // X fragments of the wave: token rows tw + 32i + (lane & 31), columns
    // 16h .. 16h+15 of the chunk.  Token rows past T read row T-1 (their
    // outputs are not stored); columns past N read an in-bounds column and
    // are zeroed just before use.
    const int64_t tw = t0 + wave * 64;
    const int hx = lane >> 5;
    const uint16_t* xrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = tw + i * 32 + (lane & 31);
        xrow[i] = X + (t < a.T ? t : a.T - 1) * a.N + 16 * hx;
    }
    auto x_load = [&](int64_t j0, u32x4 (&xv)[2][2]) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const bool jin = j0 + 16 * hx + 8 * k < a.N;
            const int64_t off = jin ? j0 + 8 * k : a.N - 8 - 16 * hx;   // clamped in-bounds column
#pragma unroll
            for (int i = 0; i < 2; ++i) xv[i][k] = *reinterpret_cast<const u32x4*>(xrow[i] + off);
        }
    };
    auto x_zero_tail = [&](int64_t j0, u32x4 (&xv)[2][2]) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const bool jin = j0 + 16 * hx + 8 * k < a.N;
#pragma unroll
            for (int i = 0; i < 2; ++i) xv[i][k] = jin ? xv[i][k] : u32x4{0, 0, 0, 0};
        }
    };

    float16v acc[2][4];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    // The chunk count is rounded up to even so both steps of the unrolled
    // loop run unconditionally (a chunk past N decodes to zeros and its X
    // fragments are zeroed, adding exact zeros); part h takes chunks
    // c_lo .. nchunks - 1, an even run.
    const int64_t nchunks_all = ((a.N + kBK - 1) / kBK + 1) & ~int64_t(1);
    const int64_t per = ((nchunks_all / 2 + ksplit - 1) / ksplit) * 2;
    const int64_t c_lo = int64_t(h) * per;
    const int64_t nchunks = c_lo + per < nchunks_all ? c_lo + per : nchunks_all;
    auto step = [&](int64_t c, u32x4 (&xc)[2][2], u32x4 (&xn)[2][2], const u32x4& ms, u32x4& ml) {
        const int cur = int(c & 1), nxt = cur ^ 1;
        if ((c + 1) * kBK > a.N) x_zero_tail(c * kBK, xc);
        x_load((c + 1) * kBK, xn);
        d.map_load((c + 3) * kBK, ml);
        bf16x8 bfr[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[ks][j] = *reinterpret_cast<const bf16x8*>(Ws + (cur * kTN + j * 32 + (lane & 31)) * kLd + 16 * hx +
                                                              8 * ks);
        // past the last chunk: unused, harmless
        d.decode(nxt, (c + 1) * kBK, Ws + (nxt * kTN + o_d) * kLd + jseg);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xc[i][ks]),
                                                                        bfr[ks][j], acc[i][j], 0, 0, 0);
        // interleave: each MFMA followed by a share of the decode
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, D::kSchedLds, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, D::kSchedValu, 0);  // VALU
        }
        if (c + 2 < nchunks) d.map_store(cur, ms);   // chunk c+2 into the buffer chunk c's decode has left
        __syncthreads();
    };

    u32x4 xA[2][2], xB[2][2], mA, mB;
    {   // prologue: slices of chunks c_lo and c_lo+1 in LDS, W_hat and X of chunk c_lo, slices of c_lo+2 in mA
        u32x4 m0, m1;
        d.map_load(c_lo * kBK, m0);
        d.map_store(0, m0);
        d.map_load((c_lo + 1) * kBK, m1);
        x_load(c_lo * kBK, xA);   // before mA, the order of every step's loads
        d.map_load((c_lo + 2) * kBK, mA);
        __syncthreads();   // tables and slices of chunk c_lo
        d.decode(0, c_lo * kBK, Ws + o_d * kLd + jseg);
        d.map_store(1, m1);
        __syncthreads();
    }
    for (int64_t c = c_lo; c < nchunks; c += 2) {
        step(c, xA, xB, mA, mB);
        step(c + 1, xB, xA, mB, mA);
    }
    // D[row][col]: row = 8*(v/4) + 4*(lane/32) + v%4 (token), col = lane%32 (output)
    float* Yo = h == 0 ? a.Y : part + size_t(h - 1) * size_t(a.T) * size_t(a.M);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t col = o0 + j * 32 + (lane & 31);
        float sc = 1.0f;
        if constexpr (D::kScaled) sc = col < a.M ? d.out_scale(col) : 0.0f;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = tw + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < a.T && col < a.M) {
                    if constexpr (D::kScaled)
                        Yo[row * a.M + col] = acc[i][j][v] * sc;
                    else
                        Yo[row * a.M + col] = acc[i][j][v];
                }
            }
    }
}

namespace {
// Y += part[0] + part[1] + ... (nparts buffers of n floats), in part order.
__global__ __launch_bounds__(256) void dgemm_add_kernel(float* Y, const float* part, int64_t n, uint32_t nparts) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    // 16-byte accesses when every part starts 16 bytes aligned (n % 4 == 0)
    const int64_t n4 = n % 4 == 0 ? n / 4 : 0, stride = int64_t(gridDim.x) * 256;
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += stride) {
        f32x4 y = reinterpret_cast<const f32x4*>(Y)[i];
        for (uint32_t p = 0; p < nparts; ++p) y += reinterpret_cast<const f32x4*>(part + size_t(p) * size_t(n))[i];
        reinterpret_cast<f32x4*>(Y)[i] = y;
    }
    for (int64_t i = 4 * n4 + int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
        float y = Y[i];
        for (uint32_t p = 0; p < nparts; ++p) y += part[size_t(p) * size_t(n) + i];
        Y[i] = y;
    }
}
}  // namespace

// Compute units of the current device (256 when none answers).
inline int64_t device_cus() {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                  hipSuccess || ncu <= 0)
        return 256;
    return ncu;
}

// K split of a launch of `tiles` workgroups (one per CU) over N columns: 2
// or 4 while that many times the tiles still fit one round and every part
// keeps at least 8 chunks; 1 otherwise.
inline uint32_t ksplit_for(int64_t tiles, int64_t N, int64_t ncu) {
    const int64_t nchunks = ((N + kBK - 1) / kBK + 1) & ~int64_t(1);
    uint32_t k = 1;
    while (k < 4 && tiles * 2 * k <= ncu && nchunks >= 16 * int64_t(k)) k *= 2;
    return k;
}

// Bytes of the parts h > 0 of a K-split launch: (ksplit - 1) x T x M floats.
inline size_t ksplit_bytes(uint32_t ksplit, int64_t T, int64_t M) {
    return ksplit > 1 ? align256(size_t(ksplit - 1) * size_t(T) * size_t(M) * sizeof(float)) : 0;
}

// The add of a K-split launch's parts (after it, on the same stream).
inline sketch_status launch_ksplit_add(float* Y, const float* part, int64_t T, int64_t M, uint32_t ksplit,
                                       hipStream_t st) {
    const int64_t n = T * M;
    int64_t grid = (n / 4 + 255) / 256;
    grid = grid < 1 ? 1 : grid > 8192 ? 8192 : grid;
    dgemm_add_kernel<<<unsigned(grid), 256, 0, st>>>(Y, part, n, ksplit - 1);
    return launch_status();
}

}  // namespace dgemm
}  // namespace sketch

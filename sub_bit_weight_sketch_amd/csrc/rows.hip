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
// NR > 0: the row count is NR (rows ignored), so every row's slice and
// gathers are issued before the first compare.
template <int RULE, int NR = 0>
__device__ inline void pick8(const uint16_t* tab, const uint16_t* idx, int64_t L, int64_t l0, uint32_t rows,
                             uint32_t (&h)[8]) {
    if constexpr (NR > 0) {
        uint32_t v[NR][8];
#pragma unroll
        for (int rho = 0; rho < NR; ++rho) {
            const u32x4 kv = *reinterpret_cast<const u32x4*>(idx + int64_t(rho) * L + l0);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[rho][e] = tab[(kv[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            h[e] = v[0][e];
            float bm = __builtin_fabsf(f16_bits_to_f32(h[e]));
#pragma unroll
            for (int rho = 1; rho < NR; ++rho) {
                const float m = __builtin_fabsf(f16_bits_to_f32(v[rho][e]));
                if (RULE == SKETCH_ABSMIN ? m > bm : m < bm) {
                    h[e] = v[rho][e];
                    bm = m;
                }
            }
        }
        return;
    }
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
// (the header is cleared here and written by a launch after this one)
__global__ void rows_proj_kernel(ProjHeader* hdr, uint16_t* idx, int64_t L, uint32_t rows, uint32_t Bgr,
                                 uint32_t seed) {
    const int64_t e = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e == 0) *hdr = ProjHeader{0, 0, 0, 0, 0, 0, {0, 0}};
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
};

// One wave per weight row: a workgroup of kRowsThreads threads takes
// kGemvRowsPerWg rows of one row block, whose table it stages in LDS.  Lane
// c walks the 8-column chunks c, c + 64, ... of its row: one 16-byte slice
// of each sketch row's forward map, 8 gathers per sketch row from LDS and
// the pick give 8 decoded weights, which multiply x[t][j .. j+7] (one
// 16-byte load per token) into the token's partial sum.  The 64 partial
// sums of a row are added by a fixed xor butterfly (deterministic).  VEC:
// N % 8 == 0; otherwise one weight at a time.
constexpr uint32_t kGemvRowsPerWg = kRowsThreads / 64;
constexpr int kRowsAhead = 4;   // 8-column chunks per lane whose loads go out together

template <int XDT, int RULE, bool VEC>
__global__ __launch_bounds__(kRowsThreads) void rows_gemv_kernel(RowsGemvArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint16_t tab[];   // [Bg]
    const uint32_t rgroups = (a.R + kGemvRowsPerWg - 1) / kGemvRowsPerWg;
    const int64_t b = blockIdx.x / rgroups;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t r = (blockIdx.x % rgroups) * kGemvRowsPerWg + (threadIdx.x >> 6);
    for (uint32_t q = threadIdx.x; q < a.Bg; q += kRowsThreads) tab[q] = a.S[b * a.Bg + q];
    __syncthreads();
    if (r >= a.R) return;   // whole waves; no barrier follows
    const bool ok = rows_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed, a.rows);
    const int64_t L = int64_t(a.R) * a.N;
    float acc[kRowsMaxTok];
#pragma unroll
    for (int t = 0; t < kRowsMaxTok; ++t) acc[t] = 0.0f;
    if (ok) {
        if constexpr (VEC) {
            // kRowsAhead chunks per round: the forward-map slices of the
            // first two sketch rows and the first token's x go out together
            // (unconditional loads; chunks past the row re-read the round's
            // first one and are skipped); further sketch rows load in the pick
            const int64_t rowoff = int64_t(r) * a.N;
            for (int64_t j0 = int64_t(lane) * 8; j0 < a.N; j0 += kRowsAhead * 64 * 8) {
                u32x4 kv[kRowsAhead][2];
                float x0[kRowsAhead][8];
#pragma unroll
                for (int u = 0; u < kRowsAhead; ++u) {
                    const int64_t j = j0 + u * 64 * 8 < a.N ? j0 + u * 64 * 8 : j0;
                    kv[u][0] = *reinterpret_cast<const u32x4*>(a.idx + rowoff + j);
                    kv[u][1] = *reinterpret_cast<const u32x4*>(a.idx + (a.rows > 1 ? L : 0) + rowoff + j);
                    load8_f32<XDT>(a.X, a.t0 * a.N + j, x0[u]);
                }
#pragma unroll
                for (int u = 0; u < kRowsAhead; ++u) {
                    const int64_t j = j0 + u * 64 * 8;
                    if (j < a.N) {
                        uint32_t h[8];
                        float bm[8];
                        for (uint32_t rho = 0; rho < a.rows; ++rho) {
                            const u32x4 kr = rho < 2 ? kv[u][rho]
                                                     : *reinterpret_cast<const u32x4*>(a.idx + int64_t(rho) * L + rowoff + j);
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const uint32_t v = tab[(kr[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu];
                                const float m = __builtin_fabsf(f16_bits_to_f32(v));
                                if (rho == 0 || (RULE == SKETCH_ABSMIN ? m > bm[e] : m < bm[e])) {
                                    h[e] = v;
                                    bm[e] = m;
                                }
                            }
                        }
                        float w[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = f16_bits_to_f32(h[e]);
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[0] += w[e] * x0[u][e];
#pragma unroll
                        for (int t = 1; t < kRowsMaxTok; ++t)
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
                const float w = f16_bits_to_f32(pick<RULE>(tab, a.idx, L, int64_t(r) * a.N + j, a.rows));
#pragma unroll
                for (int t = 0; t < kRowsMaxTok; ++t)
                    if (uint32_t(t) < a.ntok) acc[t] += w * load_elem<XDT>(a.X, (a.t0 + t) * a.N + j);
            }
        }
    }
    float mine = 0.0f;   // lane t keeps token t's sum
#pragma unroll
    for (int t = 0; t < kRowsMaxTok; ++t) {
        if (uint32_t(t) >= a.ntok) break;
        float v = acc[t];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
        if (lane == uint32_t(t)) mine = v;
    }
    if (lane < a.ntok) a.Y[(a.t0 + lane) * a.M + b * a.R + r] = ok ? mine : __builtin_nanf("");
}

// ------------------------------------------------------------ GEMM (prefill)
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));
constexpr int kRThreads = 512;     // 8 waves: two per SIMD
constexpr int kRTM = kRThreads;    // tokens per tile (8 waves x 64)
constexpr int kRTN = 128;          // outputs per tile
constexpr int kRBK = 32;           // columns per K-chunk
constexpr int kRLd = kRBK + 8;     // W_hat LDS row stride (elements)
constexpr int kRMapMax = 256;      // 16-byte forward-map slices per chunk (R * rows * 4): one per thread

struct RowsGemmArgs {
    const uint16_t* S;
    const uint16_t* idx;
    const ProjHeader* hdr;
    const uint16_t* X;   // [T][N] bf16 bits
    float* Y;
    int64_t T, M, N, nb;
    uint32_t R, Bg, seed, rows, tiles_m;
};

// 512 tokens x 128 outputs per workgroup; wave w owns tokens 64w .. 64w+63
// and all 128 outputs (2 x 4 MFMA 32x32x16 bf16, fp32 accumulate).  X is
// the bulk of the memory traffic (it is read once per 128 outputs), and a
// load instruction whose lanes span 32 token rows costs about one cycle per
// cache line it touches, so the tile is as wide in outputs as the registers
// allow.  Eight waves (two per SIMD, one workgroup per CU) share each
// decoded W_hat chunk, so a decoded weight feeds 512 tokens: each thread
// decodes 8 columns of one output row per chunk (256 tokens per tile with
// 16 columns per thread measured 178-185 us on 2048 x 4096 x 4096 with two
// sketch rows, 512 tokens 165-170 us; four rows 249 -> 201 us).
//   * The tables of the tile's row blocks are staged in LDS once.
//   * K runs in 32-column chunks.  For chunk c the MFMAs read W_hat[c] from
//     LDS and X[c] from registers; meanwhile the workgroup decodes chunk c+1
//     into the other W_hat buffer (per weight, one gather per sketch row and
//     the pick, binary16 -> bfloat16: exact for buckets of bfloat16 weights),
//     X[c+1] is loaded into registers, the forward-map slices of chunk c+3
//     (R * rows * 64 bytes) are loaded into registers and those of chunk c+2,
//     loaded one chunk earlier, are stored to LDS.  Each wait is thus for
//     loads issued a whole chunk before; one barrier per chunk.
//   * k order inside a chunk: lane (m, h) of an A fragment holds, at MFMA
//     step ks, columns 16h + 8ks .. 16h + 8ks + 7 of its token, so a lane
//     reads its 32 contiguous bytes of X with two 16-byte loads; B fragments
//     read W_hat at the same columns (the sum over k is the same).
template <int RULE, int NR>
__global__ __launch_bounds__(kRThreads, 1) void rows_gemm_kernel(RowsGemmArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    uint16_t* Ws = reinterpret_cast<uint16_t*>(lds_raw);           // [2][kRTN][kRLd]
    const uint32_t mslices = a.R * a.rows * 4;                      // 16-byte slices per chunk (<= 256)
    uint16_t* Ms = Ws + 2 * kRTN * kRLd;                            // [2][rows][R][kRBK]
    uint16_t* Ss = Ms + 2 * mslices * 8;                            // tables of the tile's blocks
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t tile_m = blockIdx.x % a.tiles_m, tile_t = blockIdx.x / a.tiles_m;
    const int64_t o0 = tile_m * kRTN, t0 = tile_t * kRTM;
    const int64_t L = int64_t(a.R) * a.N;

    if (!rows_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed, a.rows)) {   // uniform: NaN tile, nothing else read
        for (int u = tid; u < kRTM * kRTN; u += kRThreads) {
            const int64_t t = t0 + u / kRTN, o = o0 + u % kRTN;
            if (t < a.T && o < a.M) a.Y[t * a.M + o] = __builtin_nanf("");
        }
        return;
    }

    // tables of blocks bA .. bB
    const int64_t bA = o0 / a.R;
    int64_t bB = (o0 + kRTN - 1) / a.R;
    if (bB > a.nb - 1) bB = a.nb - 1;
    const int64_t nh = (bB - bA + 1) * int64_t(a.Bg);
    if (((bA * a.Bg) & 7) == 0 && (nh & 7) == 0) {
        for (int64_t e = int64_t(tid) * 8; e < nh; e += kRThreads * 8)
            *reinterpret_cast<u32x4*>(Ss + e) = *reinterpret_cast<const u32x4*>(a.S + bA * a.Bg + e);
    } else {
        for (int64_t e = tid; e < nh; e += kRThreads) Ss[e] = a.S[bA * a.Bg + e];
    }

    // forward-map slices of a chunk: slice q = (rho, r, piece), 8 columns
    // each, at most one per thread.  Every thread issues its load
    // unconditionally from a clamped (in-bounds) address, so the wait counters
    // see the same loads on every path and no load sits alone in a branch
    // waiting for its data; a clamped slice holds valid indices and is not
    // used (threads past the slice count do not store; columns past N decode
    // to 0).
    const uint32_t mq = uint32_t(tid) < mslices ? uint32_t(tid) : mslices - 1;
    const uint32_t mpc = (mq & 3) * 8;
    const uint32_t moff = ((mq >> 2) / a.R) * uint32_t(L) + ((mq >> 2) % a.R) * uint32_t(a.N) + mpc;
    auto map_load = [&](int64_t j0, u32x4& mv) {
        const bool in = j0 + mpc < a.N;
        mv = *reinterpret_cast<const u32x4*>(a.idx + (in ? int64_t(moff) + j0 : int64_t(moff) - mpc + a.N - 8));
    };
    auto map_store = [&](int buf, const u32x4& mv) {
        if (uint32_t(tid) < mslices) *reinterpret_cast<u32x4*>(Ms + (buf * mslices + tid) * 8) = mv;
    };

    // decode assignment: output row o_d of the tile, columns jseg .. jseg+7 of the chunk
    const int o_d = tid >> 2, jseg = (tid & 3) * 8;
    const int64_t orow = o0 + o_d;
    const bool orow_ok = orow < a.M;
    const uint32_t r_d = orow_ok ? uint32_t(orow % a.R) : 0;
    const uint16_t* Sblk = Ss + (orow_ok ? (orow / a.R - bA) * int64_t(a.Bg) : 0);
    // Straight-line: the picks run from in-bounds data whatever the row and
    // column (Sblk and the staged slices are valid), then a select zeroes
    // rows past M and columns past N, so the decode shares one basic block
    // with the MFMAs it is interleaved with.
    auto decode = [&](int buf, int64_t j0) {
        uint32_t pk[4];
        uint32_t h[8];
        pick8<RULE, NR>(Sblk, Ms + buf * mslices * 8, int64_t(a.R) * kRBK, int64_t(r_d) * kRBK + jseg, a.rows, h);
        const bool use = orow_ok && j0 + jseg < a.N;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t v = (__float_as_uint(f16_bits_to_f32(h[2 * e])) >> 16) |
                               (__float_as_uint(f16_bits_to_f32(h[2 * e + 1])) & 0xFFFF0000u);
            pk[e] = use ? v : 0u;
        }
        *reinterpret_cast<u32x4*>(Ws + (buf * kRTN + o_d) * kRLd + jseg) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    };

    // X fragments of the wave: token rows tw + 32i + (lane & 31), columns 16h .. 16h+15
    const int64_t tw = t0 + wave * 64;
    const int hx = lane >> 5;
    // Token rows past T read row T-1 (their outputs are not stored); columns
    // past N read an in-bounds column and are zeroed just before use.
    const uint16_t* xrow[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int64_t t = tw + i * 32 + (lane & 31);
        xrow[i] = a.X + (t < a.T ? t : a.T - 1) * a.N + 16 * hx;
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
    // columns past N in the last chunk are zeroed before use (uniform test)
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

    // One K-chunk.  Register sets alternate between consecutive chunks (the
    // loop below is unrolled by two), so no load result is copied, and every
    // wait is for loads issued one chunk earlier: X[c+1] is loaded into xn and
    // used by the next step; the maps of chunk c+3 are loaded into ml and
    // stored to LDS by the next step, which stores chunk c+2's from ms now.
    // The chunk count is rounded up to even so both steps of the unrolled
    // loop run unconditionally (a chunk past N decodes to zeros and its X
    // fragments are zeroed, adding exact zeros).
    const int64_t nchunks = ((a.N + kRBK - 1) / kRBK + 1) & ~int64_t(1);
    auto step = [&](int64_t c, u32x4 (&xc)[2][2], u32x4 (&xn)[2][2], const u32x4& ms, u32x4& ml) {
        const int cur = int(c & 1), nxt = cur ^ 1;
        if ((c + 1) * kRBK > a.N) x_zero_tail(c * kRBK, xc);
        // unconditional (past the last chunk the clamped addresses stay in
        // bounds), so the wait counters see the same loads on every path
        x_load((c + 1) * kRBK, xn);
        map_load((c + 3) * kRBK, ml);
        bf16x8 bfr[2][4];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                bfr[ks][j] = *reinterpret_cast<const bf16x8*>(Ws + (cur * kRTN + j * 32 + (lane & 31)) * kRLd + 16 * hx + 8 * ks);
        decode(nxt, (c + 1) * kRBK);   // past the last chunk: unused, harmless
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xc[i][ks]), bfr[ks][j],
                                                                        acc[i][j], 0, 0, 0);
        // interleave: each MFMA followed by a share of the decode
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);   // VALU
        }
        if (c + 2 < nchunks) map_store(cur, ms);   // chunk c+2 into the buffer chunk c's decode has left
        __syncthreads();
    };

    u32x4 xA[2][2], xB[2][2], mA, mB;
    {   // prologue: maps of chunks 0 and 1 in LDS, W_hat of chunk 0, X of chunk 0, maps of chunk 2 in mA
        u32x4 m0, m1;
        map_load(0, m0);
        map_store(0, m0);
        map_load(kRBK, m1);
        x_load(0, xA);   // before mA, the order of every step's loads
        map_load(2 * kRBK, mA);
        __syncthreads();   // tables and maps of chunk 0
        decode(0, 0);
        if (nchunks > 1) map_store(1, m1);
        __syncthreads();
    }
    for (int64_t c = 0; c < nchunks; c += 2) {
        step(c, xA, xB, mA, mB);
        step(c + 1, xB, xA, mB, mA);
    }
    // D[row][col]: row = 8*(v/4) + 4*(lane/32) + v%4 (token), col = lane%32 (output)
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t col = o0 + j * 32 + (lane & 31);
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = tw + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
                if (row < a.T && col < a.M) a.Y[row * a.M + col] = acc[i][j][v];
            }
        }
}

inline int64_t rows_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu > 0 ? ncu : 256;
}

inline size_t rows_gemm_table_lds(const Shape& s) {
    const int64_t nblk = (kRTN - 1) / s.R + 2;
    return size_t(nblk < s.nb ? nblk : s.nb) * size_t(s.Bg) * 2;
}

inline size_t rows_gemm_lds(const Shape& s) {
    return size_t(2 * kRTN * kRLd * 2) + size_t(2 * s.R * s.rows * 4 * 16) + rows_gemm_table_lds(s);
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
    rows_proj_kernel<<<unsigned((n + 255) / 256), 256, 0, st>>>(reinterpret_cast<ProjHeader*>(base),
                                                               reinterpret_cast<uint16_t*>(base + L.idx), s.R * s.N,
                                                               uint32_t(s.rows), uint32_t(s.Bg / s.rows), p->seed);
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    return launch_proj_header(proj, h, st);
}

bool gemm_rows_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch) {
    return p->w_dtype == SKETCH_BF16 && xdt == SKETCH_BF16 && batch > kRowsMaxTok && s.N % 8 == 0 &&
           s.R * s.rows * 4 <= kRMapMax && rows_gemm_lds(s) <= 160 * 1024;
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
        g.tiles_m = uint32_t((s.M + kRTN - 1) / kRTN);
        const int64_t grid = int64_t(g.tiles_m) * ((batch + kRTM - 1) / kRTM);
        if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
        const size_t lds = rows_gemm_lds(s);
        const bool mn = p->rule == SKETCH_ABSMIN;
#define SKETCH_ROWS_GEMM(NR)                                                                    \
    (mn ? (rows_gemm_kernel<SKETCH_ABSMIN, NR><<<unsigned(grid), kRThreads, lds, st>>>(g), 0)        \
        : (rows_gemm_kernel<SKETCH_ABSMAX, NR><<<unsigned(grid), kRThreads, lds, st>>>(g), 0))
        switch (s.rows) {
            case 2: SKETCH_ROWS_GEMM(2); break;
            case 3: SKETCH_ROWS_GEMM(3); break;
            case 4: SKETCH_ROWS_GEMM(4); break;
            default: SKETCH_ROWS_GEMM(0); break;
        }
#undef SKETCH_ROWS_GEMM
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
    const bool vec = s.N % 8 == 0;
    const int64_t grid = s.nb * ((s.R + kGemvRowsPerWg - 1) / kGemvRowsPerWg);
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    const size_t lds = size_t(s.Bg) * 2;
    for (int64_t t0 = 0; t0 < batch; t0 += kRowsMaxTok) {
        a.t0 = t0;
        a.ntok = uint32_t(batch - t0 < kRowsMaxTok ? batch - t0 : kRowsMaxTok);
#define SKETCH_ROWS_GEMV(XDT)                                                                             \
    (p->rule == SKETCH_ABSMIN                                                                             \
         ? (vec ? (rows_gemv_kernel<XDT, SKETCH_ABSMIN, true><<<unsigned(grid), kRowsThreads, lds, st>>>(a), 0)       \
                : (rows_gemv_kernel<XDT, SKETCH_ABSMIN, false><<<unsigned(grid), kRowsThreads, lds, st>>>(a), 0))     \
         : (vec ? (rows_gemv_kernel<XDT, SKETCH_ABSMAX, true><<<unsigned(grid), kRowsThreads, lds, st>>>(a), 0)       \
                : (rows_gemv_kernel<XDT, SKETCH_ABSMAX, false><<<unsigned(grid), kRowsThreads, lds, st>>>(a), 0)))
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

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
#include "dgemm.h"

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
constexpr int kRThreads = 512;     // 8 waves: two per SIMD
constexpr int kRTM = kRThreads;    // tokens per tile (8 waves x 64)
constexpr int kRTN = dgemm::kTN;   // outputs per tile
constexpr int kRBK = dgemm::kBK;   // columns per K-chunk
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

// The decoded-W_hat skeleton (dgemm.h) with 512 tokens x 128 outputs per
// workgroup: eight waves (two per SIMD, one workgroup per CU) share each
// decoded W_hat chunk, so a decoded weight feeds 512 tokens (256 tokens per
// tile with 16 columns per thread measured 178-185 us on 2048 x 4096 x 4096
// with two sketch rows, 512 tokens 165-170 us; four rows 249 -> 201 us).
// Decode policy: the tables of the tile's row blocks staged in LDS; per
// chunk the forward-map slices of every sketch row (rows x R x 4 pieces of 8
// columns); a thread decodes 8 columns of one output row, one gather per
// sketch row and the pick, binary16 -> bfloat16 (exact for buckets of
// bfloat16 weights).
template <int RULE, int NR>
struct RowsDecode {
    typedef RowsGemmArgs Args;
    static constexpr int kThreads = kRThreads, kSchedLds = 1, kSchedValu = 4;
    static constexpr bool kScaled = false;
    const Args& a;
    const int tid, jseg;
    const uint32_t mslices;   // 16-byte slices per chunk (<= 256)
    uint16_t* Ms;             // [2][rows][R][kBK]
    uint16_t* Ss;             // tables of blocks bA .. bB
    int64_t bA, bB;
    uint32_t moff, mpc;
    bool orow_ok;
    uint32_t r_d;
    const uint16_t* Sblk;

    __device__ RowsDecode(const Args& args, unsigned char* region, int tid_, int64_t o0, int o_d, int jseg_)
        : a(args), tid(tid_), jseg(jseg_), mslices(args.R * args.rows * 4) {
        Ms = reinterpret_cast<uint16_t*>(region);
        Ss = Ms + 2 * mslices * 8;
        bA = o0 / a.R;
        bB = (o0 + dgemm::kTN - 1) / a.R;
        if (bB > a.nb - 1) bB = a.nb - 1;
        // slice q = (rho, r, piece), 8 columns each, at most one per thread,
        // loaded unconditionally from a clamped (in-bounds) address; a
        // clamped slice holds valid indices and is not used (threads past
        // the slice count do not store; columns past N decode to 0)
        const int64_t L = int64_t(a.R) * a.N;
        const uint32_t mq = uint32_t(tid) < mslices ? uint32_t(tid) : mslices - 1;
        mpc = (mq & 3) * 8;
        moff = ((mq >> 2) / a.R) * uint32_t(L) + ((mq >> 2) % a.R) * uint32_t(a.N) + mpc;
        const int64_t orow = o0 + o_d;
        orow_ok = orow < a.M;
        r_d = orow_ok ? uint32_t(orow % a.R) : 0;
        Sblk = Ss + (orow_ok ? (orow / a.R - bA) * int64_t(a.Bg) : 0);
    }
    __device__ bool header_ok() const { return rows_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed, a.rows); }
    __device__ void stage() const {   // tables of blocks bA .. bB
        const int64_t nh = (bB - bA + 1) * int64_t(a.Bg);
        if (((bA * a.Bg) & 7) == 0 && (nh & 7) == 0) {
            for (int64_t e = int64_t(tid) * 8; e < nh; e += kThreads * 8)
                *reinterpret_cast<u32x4*>(Ss + e) = *reinterpret_cast<const u32x4*>(a.S + bA * a.Bg + e);
        } else {
            for (int64_t e = tid; e < nh; e += kThreads) Ss[e] = a.S[bA * a.Bg + e];
        }
    }
    __device__ void map_load(int64_t j0, u32x4& mv) const {
        const bool in = j0 + mpc < a.N;
        mv = *reinterpret_cast<const u32x4*>(a.idx + (in ? int64_t(moff) + j0 : int64_t(moff) - mpc + a.N - 8));
    }
    __device__ void map_store(int buf, const u32x4& mv) const {
        if (uint32_t(tid) < mslices) *reinterpret_cast<u32x4*>(Ms + (buf * mslices + tid) * 8) = mv;
    }
    // Straight-line: the picks run from in-bounds data whatever the row and
    // column (Sblk and the staged slices are valid), then a select zeroes
    // rows past M and columns past N, so the decode shares one basic block
    // with the MFMAs it is interleaved with.
    __device__ void decode(int buf, int64_t j0, uint16_t* dst) const {
        uint32_t pk[4];
        uint32_t h[8];
        pick8<RULE, NR>(Sblk, Ms + buf * mslices * 8, int64_t(a.R) * dgemm::kBK, int64_t(r_d) * dgemm::kBK + jseg,
                        a.rows, h);
        const bool use = orow_ok && j0 + jseg < a.N;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t v = (__float_as_uint(f16_bits_to_f32(h[2 * e])) >> 16) |
                               (__float_as_uint(f16_bits_to_f32(h[2 * e + 1])) & 0xFFFF0000u);
            pk[e] = use ? v : 0u;
        }
        *reinterpret_cast<u32x4*>(dst) = u32x4{pk[0], pk[1], pk[2], pk[3]};
    }
    __device__ float out_scale(int64_t) const { return 1.0f; }
};

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
    return dgemm::kWBytes + size_t(2 * s.R * s.rows * 4 * 16) + rows_gemm_table_lds(s);
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

// The optional workspace of the prefill product: the parts of a K split
// (0 when the tiles already fill the chip, or on the GEMV path).
size_t rows_gemm_split_bytes(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch) {
    if (!gemm_rows_supported(p, s, xdt, batch)) return 0;
    const int64_t tiles = ((s.M + kRTN - 1) / kRTN) * ((batch + kRTM - 1) / kRTM);
    return dgemm::ksplit_bytes(dgemm::ksplit_for(tiles, s.N, dgemm::device_cus()), batch, s.M);
}

sketch_status launch_matmul_rows(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                                 const void* X, sketch_dtype xdt, int64_t batch, float* Y, void* ws, size_t ws_bytes,
                                 hipStream_t st) {
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
        static_assert(kRTM == RowsDecode<SKETCH_ABSMIN, 2>::kThreads, "the kernel numbers its tiles with this token tile");
        g.tiles_m = uint32_t((s.M + kRTN - 1) / kRTN);
        const int64_t tiles = int64_t(g.tiles_m) * ((batch + kRTM - 1) / kRTM);
        // K split when the caller's workspace holds its parts
        const uint32_t k = dgemm::ksplit_for(tiles, s.N, dgemm::device_cus());
        const size_t need = dgemm::ksplit_bytes(k, batch, s.M);
        const uint32_t ksplit = need > 0 && ws && !(reinterpret_cast<uintptr_t>(ws) & 15u) && ws_bytes >= need ? k : 1u;
        float* part = ksplit > 1 ? static_cast<float*>(ws) : nullptr;
        const int64_t grid = tiles * ksplit;
        if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
        const size_t lds = rows_gemm_lds(s);
        const bool mn = p->rule == SKETCH_ABSMIN;
#define SKETCH_ROWS_GEMM(NR)                                                                                       \
    (mn ? (dgemm::dgemm_kernel<RowsDecode<SKETCH_ABSMIN, NR>><<<unsigned(grid), kRThreads, lds, st>>>(g, g.tiles_m, \
                                                                                                     ksplit, part),  \
           0)                                                                                                      \
        : (dgemm::dgemm_kernel<RowsDecode<SKETCH_ABSMAX, NR>><<<unsigned(grid), kRThreads, lds, st>>>(g, g.tiles_m, \
                                                                                                     ksplit, part),  \
           0))
        switch (s.rows) {
            case 2: SKETCH_ROWS_GEMM(2); break;
            case 3: SKETCH_ROWS_GEMM(3); break;
            case 4: SKETCH_ROWS_GEMM(4); break;
            default: SKETCH_ROWS_GEMM(0); break;
        }
#undef SKETCH_ROWS_GEMM
        if (ksplit == 1) return launch_status();
        if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
        return dgemm::launch_ksplit_add(Y, part, batch, s.M, ksplit, st);
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

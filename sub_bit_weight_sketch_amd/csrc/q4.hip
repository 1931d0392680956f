// q4.hip -- products and decode of the 4-bit bucket sketch.
//
// "Resumen Técnico" › Resultados: 0.5 bits per weight is reached combined
// with 4-bit quantization.  Readings (the pages give no formulas): a block
// has Bg = R*N*bpw/4 buckets (8 weights per bucket at 0.5 bpw), each a signed
// code q in [-7, 7], and one binary16 scale s; W_hat[i][j] = q * s with q the
// code of bucket k((i % R)*N + j), k the binary16 sketch's hash for Bg
// buckets (its projection's forward map).  The encoder is encode.hip's 4-bit
// mode.  Tables buffer: codes two per byte (even bucket in the low nibble),
// block b at byte b*Bg/2, then the scales (binary16 [nb]) at
// align256(nb*Bg/2).
//
// Every product applies the block's scale once per output: the codes are
// exact small integers, so the bf16 matrix cores multiply them exactly and
// the fp32 accumulators are scaled in the epilogue.  Prefill batches run on
// the binary16 sketch's tile kernel (gemm.hip: codes staged as bfloat16
// table words, gathered straight into MFMA fragments) where it applies;
// the decoded-W_hat kernel (dgemm.h, with the decode policy below), which
// decodes each weight of a chunk into LDS, takes the other shapes.
#include "common.h"
#include "dgemm.h"

namespace sketch {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQThreads = 256;
constexpr int kQMaxTok = 16;   // tokens per GEMV pass
constexpr int kQAhead = 4;     // 8-column chunks per lane whose loads go out together

__device__ inline bool q4_header_ok(const ProjHeader* h, uint32_t R, int64_t N, uint32_t Bg, uint32_t seed) {
    return h->magic == kProjMagic && h->version == kProjVersion && h->R == R && h->N == uint32_t(N) && h->Bg == Bg &&
           h->seed == seed;
}

// Signed code of bucket k in a block's packed codes.
__device__ inline int q4_code(const uint8_t* codes, uint32_t k) {
    const uint32_t nib = (uint32_t(codes[k >> 1]) >> ((k & 1u) * 4u)) & 0xFu;
    return int(nib << 28) >> 28;
}

struct Q4Args {
    const uint8_t* codes;     // [nb][Bg/2]
    const uint16_t* scales;   // [nb] binary16
    const uint16_t* idx;      // forward map [R*N] (projection)
    const ProjHeader* hdr;
    const void* X;
    float* Y;
    int64_t T, M, N, nb, t0;
    uint32_t R, Bg, seed, ntok;
};

// ------------------------------------------------------------------ GEMV
constexpr uint32_t kQRowsPerWg = kQThreads / 64;

// One wave per weight row: a workgroup takes 4 rows of one block and stages
// its Bg/2 bytes of codes in LDS.  Lane c walks the 8-column chunks c,
// c + 64, ...: one 16-byte forward-map slice, 8 byte gathers and nibble
// selects give 8 codes, which multiply x[t][j .. j+7] into the token's
// partial sum; a fixed xor butterfly adds the 64 partial sums and the block
// scale multiplies the result once.
template <int XDT, bool VEC>
__global__ __launch_bounds__(kQThreads) void q4_gemv_kernel(Q4Args a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t cod[];   // [Bg/2]
    const uint32_t rgroups = (a.R + kQRowsPerWg - 1) / kQRowsPerWg;
    const int64_t b = blockIdx.x / rgroups;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t r = (blockIdx.x % rgroups) * kQRowsPerWg + (threadIdx.x >> 6);
    const bool ok = q4_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed);
    const uint32_t nbytes = a.Bg / 2;
    const uint8_t* src = a.codes + b * int64_t(nbytes);
    for (uint32_t q = threadIdx.x; q < nbytes; q += kQThreads) cod[q] = src[q];
    __syncthreads();
    if (r >= a.R) return;   // whole waves; no barrier follows
    float acc[kQMaxTok];
#pragma unroll
    for (int t = 0; t < kQMaxTok; ++t) acc[t] = 0.0f;
    if (ok) {
        const uint16_t* Ir = a.idx + int64_t(r) * a.N;
        if constexpr (VEC) {
            // kQAhead chunks per round: their forward-map slices and the
            // first token's x go out together (unconditional loads; chunks
            // past the row re-read the round's first one and are skipped),
            // so a row takes N / (512 kQAhead) memory round trips, not N / 512
            for (int64_t j0 = int64_t(lane) * 8; j0 < a.N; j0 += kQAhead * 64 * 8) {
                u32x4 kv[kQAhead];
                float x0[kQAhead][8];
#pragma unroll
                for (int u = 0; u < kQAhead; ++u) {
                    const int64_t j = j0 + u * 64 * 8 < a.N ? j0 + u * 64 * 8 : j0;
                    kv[u] = *reinterpret_cast<const u32x4*>(Ir + j);
                    load8_f32<XDT>(a.X, a.t0 * a.N + j, x0[u]);
                }
#pragma unroll
                for (int u = 0; u < kQAhead; ++u) {
                    const int64_t j = j0 + u * 64 * 8;
                    if (j < a.N) {
                        float w[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[e] = float(q4_code(cod, (kv[u][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu));
#pragma unroll
                        for (int e = 0; e < 8; ++e) acc[0] += w[e] * x0[u][e];
#pragma unroll
                        for (int t = 1; t < kQMaxTok; ++t)
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
                const float w = float(q4_code(cod, Ir[j]));
#pragma unroll
                for (int t = 0; t < kQMaxTok; ++t)
                    if (uint32_t(t) < a.ntok) acc[t] += w * load_elem<XDT>(a.X, (a.t0 + t) * a.N + j);
            }
        }
    }
    const float sc = f16_bits_to_f32(a.scales[b]);
    float mine = 0.0f;   // lane t keeps token t's sum
#pragma unroll
    for (int t = 0; t < kQMaxTok; ++t) {
        if (uint32_t(t) >= a.ntok) break;
        float v = acc[t];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
        if (lane == uint32_t(t)) mine = v;
    }
    if (lane < a.ntok) a.Y[(a.t0 + lane) * a.M + b * a.R + r] = ok ? mine * sc : __builtin_nanf("");
}

// ------------------------------------------------------------------ GEMM
// The decoded-W_hat skeleton (dgemm.h): 256 tokens x 128 outputs per
// workgroup, MFMAs on the exact codes as bfloat16 (small integers), the
// block scale applied per output column in the epilogue.
constexpr int kQTM = 256, kQTN = dgemm::kTN;

inline int64_t q4_tile_blocks(int64_t R, int64_t nb) {
    const int64_t n = (kQTN - 1) / R + 2;
    return n < nb ? n : nb;
}

inline size_t q4_gemm_lds(const Shape& s) {
    return size_t(dgemm::kWBytes) + size_t(2 * s.R * 4 * 16) +
           ((size_t(q4_tile_blocks(s.R, s.nb)) * size_t(s.Bg / 2) + 15) & ~size_t(15));
}

// Decode policy: the codes of the tile's row blocks staged in LDS; per
// chunk, the forward-map slices of the R rows (R x 4 pieces of 8 columns);
// a thread turns 16 columns of one output row into bfloat16 codes.
struct Q4Decode {
    typedef Q4Args Args;
    static constexpr int kThreads = 256, kSchedLds = 2, kSchedValu = 8;
    static constexpr bool kScaled = true;
    const Args& a;
    const int tid, jseg;
    const uint32_t mslices;   // 16-byte map slices per chunk (<= 256)
    uint16_t* Ms;             // [2][R][kBK]
    uint8_t* Cs;              // codes of blocks bA .. bB
    int64_t bA, bB;
    uint32_t nbytes, mpc;
    int64_t moff;
    bool orow_ok;
    uint32_t r_d;
    const uint8_t* Cblk;

    __device__ Q4Decode(const Args& args, unsigned char* region, int tid_, int64_t o0, int o_d, int jseg_)
        : a(args), tid(tid_), jseg(jseg_), mslices(args.R * 4) {
        Ms = reinterpret_cast<uint16_t*>(region);
        Cs = reinterpret_cast<uint8_t*>(Ms + 2 * mslices * 8);
        bA = o0 / a.R;
        bB = (o0 + dgemm::kTN - 1) / a.R;
        if (bB > a.nb - 1) bB = a.nb - 1;
        nbytes = a.Bg / 2;
        // slice q = (r, piece), one per thread at most, loaded from a clamped
        // address (a clamped slice holds valid indices and is not used)
        const uint32_t mq = uint32_t(tid) < mslices ? uint32_t(tid) : mslices - 1;
        mpc = (mq & 3) * 8;
        moff = int64_t(mq >> 2) * a.N + mpc;
        const int64_t orow = o0 + o_d;
        orow_ok = orow < a.M;
        r_d = orow_ok ? uint32_t(orow % a.R) : 0;
        Cblk = Cs + (orow_ok ? (orow / a.R - bA) * int64_t(nbytes) : 0);
    }
    __device__ bool header_ok() const { return q4_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed); }
    __device__ void stage() const {   // codes of blocks bA .. bB (contiguous)
        const int64_t n = (bB - bA + 1) * int64_t(nbytes);
        const uint8_t* src = a.codes + bA * int64_t(nbytes);
        if (((bA * nbytes) & 15) == 0 && (n & 15) == 0) {
            for (int64_t e = int64_t(tid) * 16; e < n; e += kThreads * 16)
                *reinterpret_cast<dgemm::u32x4*>(Cs + e) = *reinterpret_cast<const dgemm::u32x4*>(src + e);
        } else {
            for (int64_t e = tid; e < n; e += kThreads) Cs[e] = src[e];
        }
    }
    __device__ void map_load(int64_t j0, dgemm::u32x4& mv) const {
        const bool in = j0 + mpc < a.N;
        mv = *reinterpret_cast<const dgemm::u32x4*>(a.idx + (in ? moff + j0 : moff - mpc + a.N - 8));
    }
    __device__ void map_store(int buf, const dgemm::u32x4& mv) const {
        if (uint32_t(tid) < mslices) *reinterpret_cast<dgemm::u32x4*>(Ms + (buf * mslices + tid) * 8) = mv;
    }
    // straight-line (in-bounds data whatever the row and column, then a
    // select), sharing one basic block with the MFMAs it is interleaved with
    __device__ void decode(int buf, int64_t j0, uint16_t* dst) const {
        const uint16_t* mb = Ms + buf * mslices * 8 + r_d * dgemm::kBK + jseg;
        uint32_t pk[8];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            const dgemm::u32x4 kv = *reinterpret_cast<const dgemm::u32x4*>(mb + hh * 8);
            const bool use = orow_ok && j0 + jseg + hh * 8 < a.N;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                // small integers are exact in bfloat16: the top half of their float32
                const uint32_t lo = __float_as_uint(float(q4_code(Cblk, kv[e] & 0xFFFFu))) >> 16;
                const uint32_t hi = __float_as_uint(float(q4_code(Cblk, kv[e] >> 16))) & 0xFFFF0000u;
                pk[hh * 4 + e] = use ? (lo | hi) : 0u;
            }
        }
        dgemm::u32x4* d = reinterpret_cast<dgemm::u32x4*>(dst);
        d[0] = dgemm::u32x4{pk[0], pk[1], pk[2], pk[3]};
        d[1] = dgemm::u32x4{pk[4], pk[5], pk[6], pk[7]};
    }
    __device__ float out_scale(int64_t col) const { return f16_bits_to_f32(a.scales[col / a.R]); }
};

// ---------------------------------------------------------------- decode
struct Q4DecArgs {
    const uint8_t* codes;
    const uint16_t* scales;
    const uint16_t* idx;      // forward map (map form)
    const ProjHeader* hdr;    // (map form)
    void* out;
    int64_t N, nb;
    uint32_t R, Bg, seed, spans, span;
};

// One workgroup per (row block, column span).  Map form: the block's codes
// staged in LDS and each index from the forward map; HASHED: every weight's
// bucket hashed and its code read from memory.  VEC (N % 8 == 0): 8 columns
// of a row per thread (one 16-byte forward-map slice, one 16- or 32-byte
// store).  A projection of another shape gives NaN.
template <int OD, bool HASHED, bool VEC>
__global__ __launch_bounds__(kQThreads) void q4_decode_kernel(Q4DecArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t cod[];   // [Bg/2] (map form)
    const int64_t b = blockIdx.x / a.spans;
    const int64_t j0 = int64_t(blockIdx.x % a.spans) * a.span;
    const int64_t j1 = j0 + a.span < a.N ? j0 + a.span : a.N;
    const uint32_t nbytes = a.Bg / 2;
    const uint8_t* src = a.codes + b * int64_t(nbytes);
    bool ok = true;
    if constexpr (!HASHED) {
        ok = q4_header_ok(a.hdr, a.R, a.N, a.Bg, a.seed);
        for (uint32_t q = threadIdx.x; q < nbytes; q += kQThreads) cod[q] = src[q];
        __syncthreads();
    }
    const float sc = f16_bits_to_f32(a.scales[b]);
    if constexpr (VEC) {
        const uint32_t cpr = uint32_t((j1 - j0) / 8);
        for (uint32_t u = threadIdx.x; u < a.R * cpr; u += kQThreads) {
            const uint32_t r = u / cpr;
            const int64_t j = j0 + int64_t(u % cpr) * 8;
            const uint32_t l0 = uint32_t(r * a.N + j);
            float v[8];
            if (!ok) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = __builtin_nanf("");
            } else if constexpr (HASHED) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = float(q4_code(src, bucket_of(l0 + e, a.seed, a.Bg))) * sc;
            } else {
                const u32x4 kv = *reinterpret_cast<const u32x4*>(a.idx + l0);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = float(q4_code(cod, (kv[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu)) * sc;
            }
            store8_val<OD>(a.out, (b * a.R + r) * a.N + j, v);
        }
        return;
    }
    const uint32_t w = uint32_t(j1 - j0);
    for (uint32_t u = threadIdx.x; u < a.R * w; u += kQThreads) {
        const uint32_t r = u / w;
        const int64_t j = j0 + (u % w);
        const uint32_t l = uint32_t(r * a.N + j);
        float v = __builtin_nanf("");
        if (ok) {
            if constexpr (HASHED)
                v = float(q4_code(src, bucket_of(l, a.seed, a.Bg))) * sc;
            else
                v = float(q4_code(cod, a.idx[l])) * sc;
        }
        store1_val<OD>(a.out, (b * a.R + r) * a.N + j, v);
    }
}

inline int64_t q4_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu > 0 ? ncu : 256;
}

bool gemm_q4_supported(const sketch_params* p, const Shape& s, sketch_dtype xdt, int64_t batch) {
    (void)p;
    return xdt == SKETCH_BF16 && batch > kQMaxTok && s.N % 8 == 0 && s.R * 4 <= 256 && q4_gemm_lds(s) <= 160 * 1024;
}

}  // namespace

sketch_status launch_matmul_q4(const sketch_params* p, const Shape& s, const void* proj, const void* tables,
                               const void* X, sketch_dtype xdt, int64_t batch, float* Y, hipStream_t st) {
    Q4Args a;
    a.codes = static_cast<const uint8_t*>(tables);
    a.scales = reinterpret_cast<const uint16_t*>(static_cast<const char*>(tables) + q4_scales_offset(s));
    a.idx = reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + proj_layout(s.R, s.N, s.Bg).idx);
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.X = X;
    a.Y = Y;
    a.T = batch;
    a.M = s.M;
    a.N = s.N;
    a.nb = s.nb;
    a.t0 = 0;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed = p->seed;
    a.ntok = 0;
    if (gemm_tile_q4_supported(s, xdt, batch))
        return launch_gemm_tile_q4(p, s, proj, a.codes, a.scales, X, batch, Y, st);
    if (gemm_q4_supported(p, s, xdt, batch)) {
        static_assert(kQTM == Q4Decode::kThreads, "the kernel numbers its tiles with this token tile");
        const uint32_t tiles_m = uint32_t((s.M + kQTN - 1) / kQTN);
        const int64_t grid = int64_t(tiles_m) * ((batch + kQTM - 1) / kQTM);
        if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
        dgemm::dgemm_kernel<Q4Decode><<<unsigned(grid), Q4Decode::kThreads, q4_gemm_lds(s), st>>>(a, tiles_m, 1u, nullptr);
        return launch_status();
    }
    const bool vec = s.N % 8 == 0;
    const int64_t grid = s.nb * ((s.R + kQRowsPerWg - 1) / kQRowsPerWg);
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    const size_t lds = (size_t(s.Bg / 2) + 15) & ~size_t(15);
    for (int64_t t0 = 0; t0 < batch; t0 += kQMaxTok) {
        a.t0 = t0;
        a.ntok = uint32_t(batch - t0 < kQMaxTok ? batch - t0 : kQMaxTok);
#define SKETCH_QGEMV(XDT)                                                                              \
    (vec ? (q4_gemv_kernel<XDT, true><<<unsigned(grid), kQThreads, lds, st>>>(a), 0)                    \
         : (q4_gemv_kernel<XDT, false><<<unsigned(grid), kQThreads, lds, st>>>(a), 0))
        switch (xdt) {
            case SKETCH_F32: SKETCH_QGEMV(SKETCH_F32); break;
            case SKETCH_BF16: SKETCH_QGEMV(SKETCH_BF16); break;
            default: SKETCH_QGEMV(SKETCH_F16); break;
        }
#undef SKETCH_QGEMV
        if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    }
    return SKETCH_OK;
}

sketch_status launch_decode_q4(const sketch_params* p, const Shape& s, const void* proj, const void* tables,
                               void* out, sketch_dtype od, bool hashed, hipStream_t st) {
    Q4DecArgs a;
    a.codes = static_cast<const uint8_t*>(tables);
    a.scales = reinterpret_cast<const uint16_t*>(static_cast<const char*>(tables) + q4_scales_offset(s));
    a.idx = proj ? reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + proj_layout(s.R, s.N, s.Bg).idx)
                 : nullptr;
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.out = out;
    a.N = s.N;
    a.nb = s.nb;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed = p->seed;
    const int64_t want = 4 * q4_cus();
    int64_t spans = (want + s.nb - 1) / s.nb;
    const int64_t max_spans = s.N / 256 > 0 ? s.N / 256 : 1;
    spans = spans < 1 ? 1 : (spans > max_spans ? max_spans : spans);
    const bool vec = s.N % 8 == 0;
    int64_t span = (s.N + spans - 1) / spans;
    if (vec) span = (span + 7) / 8 * 8;
    spans = (s.N + span - 1) / span;
    a.spans = uint32_t(spans);
    a.span = uint32_t(span);
    const int64_t grid = s.nb * spans;
    if (grid > 0x7FFFFFFF) return SKETCH_EINVAL;
    const size_t lds = hashed ? 0 : ((size_t(s.Bg / 2) + 15) & ~size_t(15));
#define SKETCH_QDEC(OD)                                                                                  \
    (hashed ? (vec ? (q4_decode_kernel<OD, true, true><<<unsigned(grid), kQThreads, lds, st>>>(a), 0)     \
                   : (q4_decode_kernel<OD, true, false><<<unsigned(grid), kQThreads, lds, st>>>(a), 0))   \
            : (vec ? (q4_decode_kernel<OD, false, true><<<unsigned(grid), kQThreads, lds, st>>>(a), 0)    \
                   : (q4_decode_kernel<OD, false, false><<<unsigned(grid), kQThreads, lds, st>>>(a), 0)))
    switch (od) {
        case SKETCH_F32: SKETCH_QDEC(SKETCH_F32); break;
        case SKETCH_BF16: SKETCH_QDEC(SKETCH_BF16); break;
        default: SKETCH_QDEC(SKETCH_F16); break;
    }
#undef SKETCH_QDEC
    return launch_status();
}

}  // namespace sketch

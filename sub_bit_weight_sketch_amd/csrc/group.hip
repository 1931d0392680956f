// group.hip -- grouped decode product: many sketched linears, each with its
// own input vector and output, in two launches (three when tiles are split).
//
// "Resumen Técnico" › Metodología §4: W_hat = S * P^T, so each linear's
// product factorises as y[b*R + r] = sum_k S[b][k] * Z[r][k] with
// Z = P^T x (Resultados › Ablación: the matrix form equals the sequential
// one).  A decoder step multiplies several linears (each with its own x) by
// one token; launched one by one, each is far too small to keep HBM busy.
// Here the whole set is one stream of bucket tables:
//   * group_z_kernel, one workgroup per slice of one linear's buckets: x into
//     LDS, Z summed per (row, bucket) segment of the projection's inverse map
//     (ascending j), and written to the workspace as binary16 hi + lo MFMA
//     fragments (every product exact, the same split as the single-linear
//     product).  The linear's power-of-two scale bounds |Z| by N * max |x|,
//     which every workgroup of the linear derives alike from the x it holds,
//     so no workgroup waits for another;
//   * group_stream_kernel: the tables of all linears form one sequence of
//     tiles (binary16 buckets: 32 blocks, two 16-block MFMA tiles; 4-bit
//     codes: 64 blocks); every wave streams a contiguous, cost-balanced range
//     of it (planned on the host), crossing from one linear to the next
//     without a barrier.  A tile streams in chunks of 8 KiB (32 rows x 256
//     bytes, or 64 rows x 128 bytes) into registers two chunks ahead (with
//     the chunk's Z fragments, which stay in L2), through the wave's LDS
//     slot into the MFMA operand pattern, 8 (32) f16 MFMAs (Z as A, tables or
//     exactly unpacked codes as B), and the hi + lo sums of each output row
//     are scaled back and stored;
//   * with fewer tiles than waves (a single decoder layer), each tile's
//     chunks are split into pieces that different waves stream; the pieces
//     leave partial sums, which group_reduce_kernel adds in a fixed order.
// 4-bit codes (Resultados: 0.5 bpw with 4-bit quantization) take the same
// factorisation with the block scale outside the sum:
// y[b*R + r] = s_b * sum_k q[b][k] * Z[r][k].
#include <algorithm>
#include <cstring>
#include <type_traits>

#include "common.h"

namespace sketch {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kGroupMagic = 0x50524753u;   // "SGRP"
// Buckets of one Z workgroup (its slice): 256 (8 K-steps), one per thread.
// A group with fewer such slices than kZSmallBelow (one decoder layer:
// 35) takes slices of 64 buckets (binary16) or 128 (4-bit codes, whose
// fragment order spans 128 buckets), so more workgroups share the work and
// each thread sums 2 or 4 of a bucket's rows instead of all 8.
constexpr uint32_t kZSlice = 256;
constexpr uint32_t kZSlice16Small = 64, kZSliceQ4Small = 128;
constexpr uint64_t kZSmallBelow = 256;
constexpr int kStreamThreads = 256;             // 4 waves
constexpr size_t kZLds = 152 * 1024;            // LDS of group_z_kernel, at most (x: 120 KiB)
constexpr uint32_t kZRow = kZSlice + 4;         // Z row stride in floats (rows 16 bytes apart in bank order)
constexpr uint32_t kZSliceBytes = 8 * kZRow * 4; // Z of one workgroup: 8 rows x its buckets (float)
constexpr uint32_t kColLds = 24 * 1024;         // staged inverse-map columns of one workgroup, at most
constexpr int64_t kMaxWaves = 8192;             // waves of the stream launch, at most
constexpr uint32_t kTileFixedCost = 4;          // per-tile overhead, in binary16 K-steps, for the balancing
constexpr uint32_t kMaxPieces = 16;             // pieces of a split tile, at most

// Geometry of the tile stream.  A chunk is 8 KiB of tables: kTile rows of
// kRowBytes contiguous bytes, kKS K-steps of 32 buckets.
//  * binary16 buckets: a stream tile is 2 MFMA tiles of 16 blocks, a chunk
//    256 bytes (128 buckets) of each of its 32 rows;
//  * 4-bit codes: 4 MFMA tiles (64 blocks), 128 bytes (256 codes) of each
//    row, so that the Z fragments a chunk reads (one per K-step, shared by
//    the MFMA tiles) stay at the chunk's own size.  The LDS rows are padded
//    by 16 bytes: the 16 rows one MFMA operand read touches then start 4
//    banks apart and cover all 64 banks once.
template <bool Q4>
struct StreamGeo {
    static constexpr int kTB = Q4 ? 4 : 2;                        // MFMA tiles per stream tile
    static constexpr int kTile = 16 * kTB;                        // row blocks per stream tile
    static constexpr uint32_t kRowBytes = 8192 / kTile;          // bytes of a row in a chunk
    static constexpr int kKS = Q4 ? 8 : 4;                        // K-steps per chunk
    static constexpr uint32_t kPitch = kRowBytes + (Q4 ? 16 : 0); // LDS row pitch
    static constexpr uint32_t kSlot = kTile * kPitch;            // a wave's LDS slot
    static constexpr int kBlocksPerCU = Q4 ? 2 : 3;               // resident stream workgroups per CU
};

// The kernels reach the linears' buffers through pointers read from the
// plan, which the compiler cannot place in an address space by itself: as
// generic (flat) accesses every wait would also drain the LDS counter and all
// loads in flight.  These casts name them as global memory.
#define SKETCH_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ inline const SKETCH_GLOBAL T* gmem(const T* p) {
    return (const SKETCH_GLOBAL T*)(p);
}
template <class T>
__device__ inline SKETCH_GLOBAL T* gmem(T* p) {
    return (SKETCH_GLOBAL T*)(p);
}
// The plan and the scales are written by earlier launches and only read by
// the stream kernel: as constant memory, its wave-uniform reads are scalar
// loads, which leave the vector load counter to the table stream.
#define SKETCH_CONST __attribute__((address_space(4)))
template <class T>
__device__ inline const SKETCH_CONST T* cmem(const T* p) {
    return (const SKETCH_CONST T*)(p);
}

// One linear of the group, as the kernels read it.
struct alignas(16) GroupItem {
    const uint16_t* S;      // tables [nb][Bg] binary16, or 4-bit codes [nb][Bg/2] bytes
    const void* x;          // [N]
    float* y;               // [M]
    const ProjHeader* hdr;  // projection (checked by group_z_kernel)
    const uint32_t* off;    // inverse map offsets [R*Bg + 1]
    const uint16_t* cols;   // inverse map columns [R*N]
    const uint16_t* bscale; // 4-bit codes: binary16 scale per block [nb] (else null)
    uint32_t N, R, Bg, seed;
    uint32_t nb, tile0;     // row blocks; first tile in the group's tile order
    uint32_t frag0;         // first 16-byte fragment of this linear in the workspace
    uint32_t zb0;           // first Z workgroup of this linear
    uint32_t row0;          // first row of this linear among the partial sums (split tiles)
    uint32_t pad;
};
static_assert(sizeof(GroupItem) == 96, "plan layout");

// pieces: the chunks of every tile are split into this many contiguous
// pieces (1: whole tiles), each a unit of the stream's work; rows_total:
// the rows of all linears (one partial sum per row and piece); zslice: the
// buckets of one Z workgroup
struct alignas(16) GroupHeader {
    uint32_t magic, count, ntiles, nwaves;
    uint32_t nfrag, xdt, nzb, tile_blocks;
    uint32_t bucket_bits, pieces, rows_total, zslice;
};

// One Z workgroup: its linear's buffers and shape, its buckets, and the runs
// of the inverse map its buckets cover in each row: run rr starts at column
// run_lo[rr] (rounded down to a 16-byte boundary) and fills LDS pieces
// piece_end[rr-1] .. piece_end[rr] - 1 (16 bytes each).
struct alignas(16) ZRec {
    const void* x;
    const uint32_t* off;
    const uint16_t* cols;
    const ProjHeader* hdr;
    uint32_t N, R, Bg, seed;
    uint32_t item, k0, nk, frag_out;   // frag_out: first fragment written
    uint32_t run_lo[8];
    uint32_t piece_end[8];
};
static_assert(sizeof(ZRec) == 128, "plan layout");

// Plan: header | items[count] | wave_tile[nwaves + 1] (each wave's first
// unit: tile * pieces + piece) | wave_item[nwaves] | zb_item[nzb] (the linear
// of every Z workgroup) | zrec[nzb] (what every Z workgroup reads, filled on
// the device when the plan is made) | tile_item[ntiles] (the linear of
// every tile, for the sum of the pieces; only when tiles are split)
struct PlanLayout {
    size_t items, wave_tile, wave_item, zb_item, zrec, tile_item, total;
};
inline PlanLayout plan_layout(int64_t count, int64_t nwaves, uint64_t nzb, uint64_t ntile_items) {
    PlanLayout L;
    L.items = align256(sizeof(GroupHeader));
    L.wave_tile = align256(L.items + sizeof(GroupItem) * size_t(count));
    L.wave_item = align256(L.wave_tile + 4 * size_t(nwaves + 1));
    L.zb_item = align256(L.wave_item + 4 * size_t(nwaves));
    L.zrec = align256(L.zb_item + 4 * size_t(nzb));
    L.tile_item = align256(L.zrec + 128 * size_t(nzb));
    L.total = align256(L.tile_item + 4 * size_t(ntile_items));
    return L;
}

int group_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu > 0 ? ncu : 256;
}

// Waves of the streaming launch: StreamGeo::kBlocksPerCU 4-wave workgroups
// per CU, all resident at once (binary16: 3, at most 168 registers per lane
// and 32 KiB of LDS each; 4-bit codes: 2, 36 KiB each).
inline int64_t group_waves(bool q4) {
    const int per_cu = q4 ? StreamGeo<true>::kBlocksPerCU : StreamGeo<false>::kBlocksPerCU;
    return int64_t(per_cu * group_cus()) * (kStreamThreads / 64);
}

// ---------------------------------------------------------------------------
// Plan upload: the host assembles the plan in pieces of at most kPiece words
// and each piece travels as a kernel argument (nothing is allocated, and the
// upload can be captured into a graph like any launch).
// ---------------------------------------------------------------------------
constexpr int kPiece = 800;
struct PlanPiece {
    uint32_t word0, n;
    uint32_t w[kPiece];
};
__global__ void plan_write_kernel(uint32_t* plan, PlanPiece p) {
    for (uint32_t i = threadIdx.x; i < p.n; i += blockDim.x) plan[p.word0 + i] = p.w[i];
}

struct PlanWriter {
    uint32_t* dst;
    hipStream_t st;
    PlanPiece piece;
    bool failed = false;
    PlanWriter(void* d, hipStream_t s) : dst(static_cast<uint32_t*>(d)), st(s) { piece.n = 0; piece.word0 = 0; }
    void flush() {
        if (piece.n == 0) return;
        plan_write_kernel<<<1, 256, 0, st>>>(dst, piece);
        if (hipGetLastError() != hipSuccess) failed = true;
        piece.word0 += piece.n;
        piece.n = 0;
    }
    // words must be written in increasing position order
    void put(size_t word, uint32_t v) {
        if (piece.n > 0 && word != size_t(piece.word0) + piece.n) flush();
        if (piece.n == 0) piece.word0 = uint32_t(word);
        piece.w[piece.n++] = v;
        if (piece.n == kPiece) flush();
    }
    // the words of an object of any type: copied out bytewise, since reading
    // its pointer members through a uint32_t lvalue would break the aliasing
    // rules (and does break the plan at -O3)
    void put_bytes(size_t byte, const void* src, size_t nbytes) {
        const unsigned char* s = static_cast<const unsigned char*>(src);
        for (size_t i = 0; i < nbytes / 4; ++i) {
            uint32_t v;
            memcpy(&v, s + 4 * i, 4);
            put(byte / 4 + i, v);
        }
    }
};

// Raw buffer resource (base, no stride, size in bytes; dword 3 of the gfx9
// family's untyped 32-bit format).  Loads through it read zero past the
// size instead of faulting, so the stream needs no clamping.
constexpr int kBufferWord3 = 0x00020000;
__device__ inline uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
// (base and size are wave-uniform; saying so keeps the resource in scalar
// registers)
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint64_t pu = (uint64_t(uniform(uint32_t(p >> 32))) << 32) | uniform(uint32_t(p));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(pu), 0, int(uniform(bytes)), kBufferWord3);
}
constexpr int kLoadNT = 2;   // cache policy of a streamed, read-once load
// Loads at byte offset voff + soff (soff wave-uniform).  The sum goes in the
// per-lane offset operand and the scalar one stays 0: the range check that
// turns reads past the size into zeros is made on the per-lane and
// immediate offsets, so every byte offset is checked in full.
__device__ inline uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, voff + soff, 0, 0);
}
__device__ inline uint32_t buffer_load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, voff + soff, 0, 0);
}
template <int POLICY>
__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + soff, 0, POLICY));
}

// ---------------------------------------------------------------------------
// Z fragments, one workgroup of THREADS threads per slice of S = THREADS RPT
// / 8 buckets k0 .. k0 + S - 1 of one linear; thread t sums rows t / S +
// (8 / RPT) i, i < RPT, of bucket k0 + t % S.  Binary16 groups take 512
// threads (2 per bucket of a 256-bucket slice), 4-bit groups 256 (measured:
// 32 layers 113.9 -> 111.4 us binary16, 169.8 -> 172.6 us 4-bit with 512).
// frag[s*64 + kq*16 + c] = 8 buckets of column c, c = 2 rr + h: the hi
// (h = 0) or lo (h = 1) binary16 part of Z[rr][k] * su; columns of rows
// rr >= R are zero.  The 8 buckets of K-step s and lane group kq are, in
// element order e = 0..7:
//  * binary16 buckets: k = 32 s + 8 kq + e;
//  * 4-bit codes: k = 128 (s / 4) + 32 kq + 8 (s % 4) + pe(e), with
//    pe(e) = 2 (e % 4) + e / 4: the order in which the stream kernel unpacks
//    the 8 codes of one 32-bit word (the even codes, then the odd ones), and
//    the word a lane reads for K-step s of its 16-byte slice.
// ---------------------------------------------------------------------------
template <int XDT>
__device__ inline float x_at(const unsigned char* xl, uint32_t j) {
    if constexpr (XDT == SKETCH_F32)
        return reinterpret_cast<const float*>(xl)[j];
    else if constexpr (XDT == SKETCH_BF16)
        return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(xl)[j]);
    else
        return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(xl)[j]);
}

// |v| as float bits, +Inf for NaN: ordered like the magnitudes
__device__ inline uint32_t mag_bits(float v) {
    const uint32_t m = __float_as_uint(v) & 0x7FFFFFFFu;
    return m > 0x7F800000u ? 0x7F800000u : m;
}

// The record of every Z workgroup (one thread each), when the plan is made:
// the slice's runs are read from the projection's offsets once, not on
// every call.
__global__ void group_prep_kernel(const GroupItem* items, const uint32_t* zb_item, ZRec* zrec, uint32_t nzb,
                                  uint32_t zslice) {
    const uint32_t zb = blockIdx.x * blockDim.x + threadIdx.x;
    if (zb >= nzb) return;
    const GroupItem it = items[zb_item[zb]];
    ZRec r;
    r.x = it.x;
    r.off = it.off;
    r.cols = it.cols;
    r.hdr = it.hdr;
    r.N = it.N;
    r.R = it.R;
    r.Bg = it.Bg;
    r.seed = it.seed;
    r.item = zb_item[zb];
    r.k0 = (zb - it.zb0) * zslice;
    r.nk = it.Bg - r.k0 < zslice ? it.Bg - r.k0 : zslice;
    r.frag_out = it.frag0 + (zb - it.zb0) * (zslice / 32) * 64;
    // a projection of other parameters gives empty runs (its Z is NaN)
    const bool ok = it.hdr->magic == kProjMagic && it.hdr->version == kProjVersion && it.hdr->R == it.R &&
                    it.hdr->N == it.N && it.hdr->Bg == it.Bg && it.hdr->seed == it.seed;
    uint32_t end = 0;
    for (uint32_t i = 0; i < 8; ++i) {
        uint32_t lo = 0, hi = 0;
        if (ok && i < it.R) {
            lo = it.off[i * it.Bg + r.k0];
            hi = it.off[i * it.Bg + r.k0 + r.nk];
            hi = hi > lo ? hi : lo;
        }
        r.run_lo[i] = lo & ~7u;
        end += i < it.R ? (hi - r.run_lo[i] + 7) / 8 : 0u;
        r.piece_end[i] = end;
    }
    zrec[zb] = r;
}

template <int XDT, bool Q4, int RPT, int THREADS>
__global__ __launch_bounds__(THREADS) void group_z_kernel(const ZRec* zrecs, half8* frags, float* scales,
                                                          uint32_t col_lds) {
    constexpr int kZThreads = THREADS;
    constexpr uint32_t kS = THREADS * RPT / 8, kTpb = 8 / RPT;   // buckets of the slice, threads per bucket
    static_assert(kS * kTpb == THREADS && kS <= kZSlice && (!Q4 || kS % 128 == 0), "slice geometry");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ uint32_t wmax[kZThreads / 64];
    // the record, as 16-byte scalar words
    ZRec it;
    {
        const SKETCH_CONST u32x4* src = reinterpret_cast<const SKETCH_CONST u32x4*>(cmem(zrecs) + blockIdx.x);
        u32x4 w[sizeof(ZRec) / 16];
#pragma unroll
        for (int k = 0; k < int(sizeof(ZRec) / 16); ++k) w[k] = src[k];
        __builtin_memcpy(&it, w, sizeof(ZRec));
    }
    const uint32_t item = it.item, k0 = it.k0, nk = it.nk;   // nk: a multiple of 32
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr uint32_t xb = XDT == SKETCH_F32 ? 4u : 2u;
    unsigned char* xl = lds;
    // after x: the staged columns, then (once they are used) Z of the slice
    unsigned char* region = lds + ((size_t(it.N) * xb + 15) & ~size_t(15));
    float* zl = reinterpret_cast<float*>(region);   // [8][kZRow]
    const SKETCH_GLOBAL ProjHeader* hdr = gmem(it.hdr);
    // buffers of the linear (reads past their ends give zero)
    const __amdgpu_buffer_rsrc_t offr = buffer_rsrc(it.off, (it.R * it.Bg + 1) * 4);
    const __amdgpu_buffer_rsrc_t colr = buffer_rsrc(it.cols, it.R * it.N * 2);
    const __amdgpu_buffer_rsrc_t xr = buffer_rsrc(it.x, it.N * xb);
    const bool ok = hdr->magic == kProjMagic && hdr->version == kProjVersion && hdr->R == it.R && hdr->N == it.N &&
                    hdr->Bg == it.Bg && hdr->seed == it.seed;
    // One round of loads: the segment bounds of bucket k0 + tid in rows
    // 0 .. 7 (rows past R and buckets past the slice: loaded, unused), the
    // first 16-byte pieces of x and the slice's inverse-map columns.
    const uint32_t kk = uint32_t(tid) % kS, rg = uint32_t(tid) / kS;   // bucket k0 + kk, first row rg
    const uint32_t k = k0 + kk;
    uint32_t b[RPT], en[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const uint32_t sg = (rg + kTpb * uint32_t(i)) * it.Bg + k;
        b[i] = buffer_load4(offr, sg * 4, 0);
        en[i] = buffer_load4(offr, sg * 4 + 4, 0);
    }
    constexpr uint32_t kU = 8;   // x pieces per thread in the first round (8 THREADS x 16 bytes of x)
    const uint32_t nv = it.N * xb / 16;
    u32x4 vv[kU];
#pragma unroll
    for (uint32_t u = 0; u < kU; ++u) vv[u] = buffer_load16<0>(xr, uint32_t(tid) * 16, u * kZThreads * 16);
    // The columns of the slice: in each row rr the segments of buckets
    // k0 .. k0+nk-1 are one contiguous run of the inverse map (the record's
    // runs).  The runs go to LDS as 16-byte pieces (coalesced), requested
    // with x, unless together they exceed col_lds; then every column is
    // read on its own from global memory.
    uint32_t piece_base[9], run_lo[8];
    piece_base[0] = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        piece_base[i + 1] = it.piece_end[i];
        run_lo[i] = it.run_lo[i];
    }
    const uint32_t npieces = piece_base[8];
    const bool staged = npieces * 16 <= col_lds;   // uniform
    constexpr uint32_t kP = kColLds / 16 / kZThreads;   // pieces per thread, at most
    u32x4 pc[kP];
    if (staged) {
#pragma unroll
        for (uint32_t u = 0; u < kP; ++u) {
            const uint32_t p = u * kZThreads + uint32_t(tid);
            uint32_t lo = run_lo[0], first = 0;   // the run holding piece p (selects, no indexing)
#pragma unroll
            for (int r = 1; r < 8; ++r) {
                lo = p >= piece_base[r] ? run_lo[r] : lo;
                first = p >= piece_base[r] ? piece_base[r] : first;
            }
            pc[u] = buffer_load16<0>(colr, (lo + (p - first) * 8) * 2, 0);
        }
    }
    // x -> LDS (raw bits) and max |x|
    uint32_t mx = 0;
    auto take = [&](uint32_t q, const u32x4& v) {
        *reinterpret_cast<u32x4*>(xl + 16 * q) = v;
        if constexpr (XDT == SKETCH_F32) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t m = mag_bits(__uint_as_float(v[e]));
                mx = m > mx ? m : mx;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t h = (v[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                const uint32_t m = mag_bits(XDT == SKETCH_BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h));
                mx = m > mx ? m : mx;
            }
        }
    };
#pragma unroll
    for (uint32_t u = 0; u < kU; ++u) {
        const uint32_t q = u * kZThreads + uint32_t(tid);
        if (q < nv) take(q, vv[u]);
    }
    for (uint32_t q = kU * kZThreads + uint32_t(tid); q < nv; q += kZThreads)   // x beyond the first round
        take(q, buffer_load16<0>(xr, q * 16, 0));
    for (uint32_t e = nv * (16 / xb) + tid; e < it.N; e += kZThreads) {   // the tail
        float f;
        if constexpr (XDT == SKETCH_F32) {
            const uint32_t u = buffer_load4(xr, e * 4, 0);
            reinterpret_cast<uint32_t*>(xl)[e] = u;
            f = __uint_as_float(u);
        } else {
            const uint16_t u = uint16_t(buffer_load2(xr, e * 2, 0));
            reinterpret_cast<uint16_t*>(xl)[e] = u;
            f = XDT == SKETCH_BF16 ? bf16_bits_to_f32(u) : f16_bits_to_f32(u);
        }
        const uint32_t m = mag_bits(f);
        mx = m > mx ? m : mx;
    }
    unsigned char* cl = region;   // [npieces] x 16 bytes
    if (staged) {
#pragma unroll
        for (uint32_t u = 0; u < kP; ++u) {
            const uint32_t p = u * kZThreads + uint32_t(tid);
            if (p < npieces) *reinterpret_cast<u32x4*>(cl + 16 * p) = pc[u];
        }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t t = uint32_t(__shfl_xor(int(mx), o));
        mx = t > mx ? t : mx;
    }
    if (lane == 0) wmax[wave] = mx;
    __syncthreads();
    // Z[rr][k0 + kk] of the thread's rows rr < R, every sum in ascending j.
    // Columns go in batches of 8 per segment for all the thread's rows
    // together: 8 RPT independent column reads, then as many x reads, then
    // the masked sums (a chain of dependent reads per column, or per row,
    // would leave the LDS latency exposed).  Rows past R have empty segments.
    float zv[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) zv[i] = 0.0f;
    if (kk < nk) {
        const uint16_t* cls = reinterpret_cast<const uint16_t*>(cl);
        const uint32_t n1 = it.N - 1;
        uint32_t len[RPT], at[RPT], most = 0;
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const uint32_t rr = rg + kTpb * uint32_t(i);
            uint32_t pbr = piece_base[0], rlo = run_lo[0];   // the row's run (selects, no indexing)
#pragma unroll
            for (int r = 1; r < 8; ++r) {
                pbr = rr == uint32_t(r) ? piece_base[r] : pbr;
                rlo = rr == uint32_t(r) ? run_lo[r] : rlo;
            }
            len[i] = rr < it.R ? en[i] - b[i] : 0u;
            at[i] = pbr * 8 + (b[i] - rlo);
            most = len[i] > most ? len[i] : most;
        }
        // One batch: the columns of positions c0 .. c0+7 of every segment
        // (past a segment's end: its first column, masked), then x, then the
        // sums.  Staged and unstaged columns take separate loops: as one
        // select, the compiler would issue the global reads in both cases.
        auto batch = [&](uint32_t c0, const uint32_t (&j)[RPT][8]) {
            float v[RPT][8];
#pragma unroll
            for (int i = 0; i < RPT; ++i)
#pragma unroll
                for (int u = 0; u < 8; ++u) v[i][u] = x_at<XDT>(xl, j[i][u] < n1 ? j[i][u] : n1);
#pragma unroll
            for (int i = 0; i < RPT; ++i)
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    if (c0 + uint32_t(u) < len[i]) zv[i] += v[i][u];
        };
        if (staged) {
            for (uint32_t c0 = 0; c0 < most; c0 += 8) {
                uint32_t j[RPT][8];
#pragma unroll
                for (int i = 0; i < RPT; ++i)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t c = c0 + uint32_t(u) < len[i] ? c0 + uint32_t(u) : 0u;
                        j[i][u] = cls[at[i] + c];
                    }
                batch(c0, j);
            }
        } else {
            for (uint32_t c0 = 0; c0 < most; c0 += 8) {
                uint32_t j[RPT][8];
#pragma unroll
                for (int i = 0; i < RPT; ++i)
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const uint32_t c = c0 + uint32_t(u) < len[i] ? c0 + uint32_t(u) : 0u;
                        j[i][u] = buffer_load2(colr, (b[i] + c) * 2, 0);
                    }
                batch(c0, j);
            }
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) zv[i] = ok ? zv[i] : __builtin_nanf("");
    }
    __syncthreads();   // the columns are used: Z takes their place
    if (kk < nk) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const uint32_t rr = rg + kTpb * uint32_t(i);
            if (rr < it.R) zl[rr * kZRow + kk] = zv[i];
        }
    }
    // |Z| <= N max|x| < 2^(ilogb(max|x|) + 1 + ceil(log2 N)): the power of two
    // su brings that bound to 2^15 (none for a zero or non-finite x; at most
    // 2^+-120)
    uint32_t mall = wmax[0];
#pragma unroll
    for (int w = 1; w < kZThreads / 64; ++w) mall = wmax[w] > mall ? wmax[w] : mall;
    const float m = __uint_as_float(mall);
    int e = 0;
    if (m <= 3.402823466e38f && m > 0.0f) {
        const int cl = it.N > 1 ? 32 - __builtin_clz(it.N - 1) : 0;
        e = 14 - ilogbf(m) - cl;
        e = e > 120 ? 120 : e < -120 ? -120 : e;
    }
    const float su = ldexpf(1.0f, e);
    if (k0 == 0 && tid == 0) scales[item] = ldexpf(1.0f, -e);
    __syncthreads();
    // fragments of K-steps k0/32 .. (k0 + nk)/32 - 1
    const uint32_t nf = (nk / 32) * 64;
    half8* fr = frags + it.frag_out;
    for (uint32_t f = tid; f < nf; f += kZThreads) {
        const uint32_t s = f >> 6, kq = (f >> 4) & 3, c = f & 15, rr = c >> 1, h = c & 1;
        half8 out = half8{};
        if (rr < it.R) {
            const float* zr = Q4 ? zl + rr * kZRow + (s >> 2) * 128 + kq * 32 + (s & 3) * 8
                                 : zl + rr * kZRow + s * 32 + kq * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = zr[Q4 ? 2 * (i & 3) + (i >> 2) : i] * su;
                const _Float16 hi = static_cast<_Float16>(v);
                // a non-finite value keeps its hi part only (Inf stays Inf)
                const float lo = __builtin_isfinite(v) ? v - static_cast<float>(hi) : 0.0f;
                out[i] = h ? static_cast<_Float16>(lo) : hi;
            }
        }
        fr[f] = out;
    }
}

// ---------------------------------------------------------------------------
// The tile stream.  A stream tile is kTB MFMA tiles of 16 row blocks; a chunk
// is kKS K-steps of it, 8 KiB of tables: kTile rows x kRowBytes contiguous
// bytes.  Each Z fragment of the chunk feeds kTB MFMAs, so the fragments
// read from L2 are 1/kTB of the table bytes (binary16: 1/2; 4-bit codes,
// whose K-step is a quarter of the bytes: 1).
// ---------------------------------------------------------------------------
struct StreamArgs {
    const GroupItem* items;
    const uint32_t* wave_tile;   // [nwaves + 1]: first unit (tile * pieces + piece) of every wave
    const uint32_t* wave_item;   // [nwaves]
    const half8* frags;
    const float* scales;
    float* partial;              // [pieces][rows_total] when pieces > 1
    uint32_t count, nwaves, nfrag, pieces, rows_total;
};

// The 8 signed 4-bit codes of a 32-bit word (code i in bits 4i .. 4i+3, two's
// complement) as binary16, in the order 0, 2, 4, 6, 1, 3, 5, 7: the even and
// the odd codes each go to the low nibbles of one word's bytes, with bit 3
// flipped (q + 8 in 0 .. 15, offset binary); a byte permute pairs two of
// them with the byte 0x64 above each, i.e. the binary16 value 1024 + q + 8,
// and one packed subtraction of 1032 leaves q, exactly.
__device__ inline half8 unpack_codes(uint32_t w) {
    const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;          // codes 0, 2, 4, 6
    const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;   // codes 1, 3, 5, 7
    constexpr uint32_t kHigh = 0x64646464u;
    u32x4 p;   // byte selectors: 0-3 the low word's bytes, 4 a byte of kHigh
    p[0] = __builtin_amdgcn_perm(kHigh, lo, 0x04010400u);
    p[1] = __builtin_amdgcn_perm(kHigh, lo, 0x04030402u);
    p[2] = __builtin_amdgcn_perm(kHigh, hi, 0x04010400u);
    p[3] = __builtin_amdgcn_perm(kHigh, hi, 0x04030402u);
    const _Float16 b = static_cast<_Float16>(1032.0f);
    return __builtin_bit_cast(half8, p) - half8{b, b, b, b, b, b, b, b};
}

template <bool Q4>
__global__ __launch_bounds__(kStreamThreads, StreamGeo<Q4>::kBlocksPerCU) void group_stream_kernel(StreamArgs a) {
    using G = StreamGeo<Q4>;
    constexpr int kTB = G::kTB, kTile = G::kTile, kKS = G::kKS;
    constexpr uint32_t kRowBytes = G::kRowBytes, kPitch = G::kPitch;
    constexpr uint32_t kLanesPerRow = kRowBytes / 16;      // lanes that load one row of a chunk
    constexpr uint32_t kRowsPerLoad = 64 / kLanesPerRow;   // rows of one load instruction
    static_assert(kRowsPerLoad * 8 == uint32_t(kTile), "8 loads per lane cover a chunk");
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-aware numbering: the workgroups of one XCD take consecutive wave
    // ranges, so each XCD's L2 holds the fragments of its own linears
    uint32_t bid = blockIdx.x;
    if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
    const uint32_t gw = bid * (kStreamThreads / 64) + uint32_t(wave);
    if (gw >= a.nwaves) return;
    const SKETCH_CONST uint32_t* wave_tile = cmem(a.wave_tile);
    const uint32_t t_begin = wave_tile[gw], t_end = wave_tile[gw + 1];
    if (t_begin >= t_end) return;
    const SKETCH_CONST GroupItem* items = cmem(a.items);
    const SKETCH_CONST float* scales = cmem(a.scales);
    unsigned char* slot = lds + size_t(wave) * G::kSlot;
    const uint32_t n = uint32_t(lane) & 15u, qd = uint32_t(lane) >> 4;

    // what the stream reads of a linear (the rest of its plan entry is the
    // Z launch's)
    struct SItem {
        const uint16_t* S;
        float* y;
        const uint16_t* bscale;
        uint32_t R, Bg, nb, tile0, frag0, row0;
    };
    // chunk cursor: (item, tile, piece, chunk) with the item's geometry
    // cached; the piece covers chunks .. ce - 1 of its tile
    struct Cursor {
        uint32_t item, tile, piece, c, ce;
        SItem it;
    };
    auto load_item = [&](uint32_t i, SItem& it) {
        const SKETCH_CONST GroupItem* g = items + (i < a.count ? i : a.count - 1);
        it.S = g->S;
        it.y = g->y;
        it.bscale = g->bscale;
        it.R = g->R;
        it.Bg = g->Bg;
        it.nb = g->nb;
        it.tile0 = g->tile0;
        it.frag0 = g->frag0;
        it.row0 = g->row0;
    };
    auto nchunks_of = [](const SItem& it) { return (it.Bg / 32 + kKS - 1) / kKS; };
    const uint32_t pieces = a.pieces;
    // piece p of a tile: chunks p*n/pieces .. (p+1)*n/pieces - 1 (pieces <= n)
    auto enter_piece = [&](Cursor& q) {
        const uint32_t nc = nchunks_of(q.it);
        q.c = q.piece * nc / pieces;
        q.ce = (q.piece + 1) * nc / pieces;
    };
    auto advance = [&](Cursor& q) {
        if (++q.c >= q.ce) {
            if (++q.piece >= pieces) {
                q.piece = 0;
                ++q.tile;
                if (q.tile >= q.it.tile0 + (q.it.nb + kTile - 1) / kTile && q.item + 1 < a.count) {
                    ++q.item;
                    load_item(q.item, q.it);
                }
            }
            enter_piece(q);
        }
    };
    // A chunk in registers: 8 x 16 bytes per lane, rows kRowsPerLoad * i +
    // lane / kLanesPerRow of the tile, bytes kRowBytes * c + 16 (lane %
    // kLanesPerRow) .. +16 of the row; with 4-bit codes also the scale of
    // block 64 * tile + lane (one per lane, for the epilogue).
    struct Chunk {
        u32x4 v[8];
        uint32_t sc;
    };
    // One per-lane offset and a uniform one per load.  Past the end of a row
    // the bytes are the next row's, past the linear's tables they read as
    // zero: neither is used, so the loads of the next chunk go out
    // unconditionally and every wait counts them exactly.
    auto load_tables = [&](const Cursor& q, Chunk& ch) {
        const SItem& it = q.it;
        const uint32_t rowb = Q4 ? it.Bg / 2 : it.Bg * 2;   // bytes of one table row
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(it.S, it.nb * rowb);
        const uint32_t vo = (uint32_t(lane) / kLanesPerRow) * rowb + (uint32_t(lane) % kLanesPerRow) * 16;
        const uint32_t so = uniform((q.tile - it.tile0) * kTile * rowb + q.c * kRowBytes);
#pragma unroll
        for (int i = 0; i < 8; ++i) ch.v[i] = buffer_load16<kLoadNT>(rs, vo, so + uint32_t(i) * kRowsPerLoad * rowb);
        if constexpr (Q4) {
            const __amdgpu_buffer_rsrc_t bs = buffer_rsrc(it.bscale, it.nb * 2);
            ch.sc = buffer_load2(bs, uint32_t(lane) * 2, uniform((q.tile - it.tile0) * kTile * 2));
        }
    };
    // the chunk's kKS Z fragments (L2-resident: every tile of the linear
    // reads them); K-steps past the linear's read the next one's, unused
    const __amdgpu_buffer_rsrc_t frs = buffer_rsrc(a.frags, a.nfrag * 16);
    auto load_frags = [&](const Cursor& q, half8 (&f)[kKS]) {
        const uint32_t so = uniform((q.it.frag0 + q.c * kKS * 64) * 16);
#pragma unroll
        for (int i = 0; i < kKS; ++i)
            f[i] = __builtin_bit_cast(half8, buffer_load16<0>(frs, uint32_t(lane) * 16, so + uint32_t(i) * 1024));
    };

    // three chunks: q0 (being multiplied), q1 (landing), q2 (requested)
    Cursor q0;
    q0.item = cmem(a.wave_item)[gw];
    load_item(q0.item, q0.it);
    q0.tile = t_begin / pieces;
    q0.piece = t_begin % pieces;
    enter_piece(q0);
    Cursor q1 = q0;
    advance(q1);
    Cursor q2 = q1;
    advance(q2);
    Chunk ca, cb, cc;
    half8 f[kKS];
    load_tables(q0, ca);
    load_tables(q1, cb);
    float4v acc[kTB];
#pragma unroll
    for (int h = 0; h < kTB; ++h) acc[h] = float4v{0.f, 0.f, 0.f, 0.f};

    auto do_chunk = [&](const Cursor& q, const Chunk& ch) {
        // row kRowsPerLoad * i + lane / kLanesPerRow of the slot
#pragma unroll
        for (int i = 0; i < 8; ++i)
            *reinterpret_cast<u32x4*>(slot + (uint32_t(i) * kRowsPerLoad + uint32_t(lane) / kLanesPerRow) * kPitch +
                                      (uint32_t(lane) % kLanesPerRow) * 16) = ch.v[i];
        const uint32_t nst = q.it.Bg / 32;
        // K-steps past the linear's last (in its last chunk) hold other
        // bytes: both operands become zero, without a branch (a branch here
        // invites the compiler to sink the fragment loads into it and wait on
        // every load in flight)
        if constexpr (Q4) {
            // B: block 16h + n, codes of bytes 64g + 16qd .. +16 of the
            // chunk's row: word u is K-step 4g + u.  Unpacked codes are
            // always finite, so a zero Z operand alone removes a K-step; it
            // is masked with a wave-uniform bitmask (a select here becomes a
            // branch around each unpack)
            u32x4 wv[kKS / 4][kTB];
#pragma unroll
            for (int g = 0; g < kKS / 4; ++g)
#pragma unroll
                for (int h = 0; h < kTB; ++h)
                    wv[g][h] = *reinterpret_cast<const u32x4*>(slot + (16 * h + n) * kPitch + g * 64 + qd * 16);
#pragma unroll
            for (int g = 0; g < kKS / 4; ++g)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t keep = uniform(q.c * kKS + uint32_t(4 * g + u) < nst ? ~0u : 0u);
                    const half8 av = __builtin_bit_cast(half8, __builtin_bit_cast(u32x4, f[4 * g + u]) & keep);
#pragma unroll
                    for (int h = 0; h < kTB; ++h)
                        acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, unpack_codes(wv[g][h][u]), acc[h], 0, 0, 0);
                }
        } else {
#pragma unroll
            for (int s4 = 0; s4 < kKS; ++s4) {
                const bool in = q.c * kKS + uint32_t(s4) < nst;   // wave-uniform
                const half8 av = in ? f[s4] : half8{};
#pragma unroll
                for (int h = 0; h < kTB; ++h) {
                    // B: block 16h + n, buckets 32 s4 + 8 qd .. +8 of the chunk
                    half8 bv = *reinterpret_cast<const half8*>(slot + (16 * h + n) * kPitch + s4 * 64 + qd * 16);
                    bv = in ? bv : half8{};
                    acc[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, bv, acc[h], 0, 0, 0);
                }
            }
        }
        if (q.c + 1 == q.ce) {
            // lane (n, qd): rows 2qd and 2qd + 1 (hi + lo columns) of block n
            // of each MFMA tile.  A whole tile (one piece) writes y; a piece
            // of a split tile writes its unscaled partial sums, which
            // group_reduce_kernel adds in piece order and scales.
            const SItem& it = q.it;
            const float sd = scales[q.item];
            const uint32_t r0 = 2 * qd;
            const bool whole = pieces == 1;   // uniform
#pragma unroll
            for (int h = 0; h < kTB; ++h) {
                float sb = 1.0f;   // 4-bit codes: the block's scale, from lane 16h + n
                if constexpr (Q4) sb = f16_bits_to_f32(uint16_t(__shfl(int(ch.sc), 16 * h + int(n), 64)));
                const float m = whole ? sd * sb : 1.0f;
                const uint32_t blk = (q.tile - it.tile0) * kTile + 16 * h + n;
                if (blk < it.nb && r0 < it.R) {
                    const float y0 = (acc[h][0] + acc[h][1]) * m, y1 = (acc[h][2] + acc[h][3]) * m;
                    SKETCH_GLOBAL float* yp =
                        whole ? gmem(it.y + size_t(blk) * it.R + r0)
                              : gmem(a.partial + size_t(q.piece) * a.rows_total + it.row0 + size_t(blk) * it.R + r0);
                    if (r0 + 1 < it.R)
                        __builtin_nontemporal_store(float2v{y0, y1}, reinterpret_cast<SKETCH_GLOBAL float2v*>(yp));
                    else
                        *yp = y0;
                }
                acc[h] = float4v{0.f, 0.f, 0.f, 0.f};
            }
        }
    };

    // A ring of three chunk buffers: while one chunk is multiplied, the next
    // two are in flight.  The current fragments go out before the newest
    // tables, so waiting for them leaves the table stream in flight; loads
    // past the wave's range read unused (or zero) bytes.
    auto step = [&](const Chunk& cur, Chunk& req) {
        load_frags(q0, f);
        load_tables(q2, req);
        __builtin_amdgcn_sched_barrier(0);   // the loads go out here, in this order
        do_chunk(q0, cur);
        const bool more = q1.tile * pieces + q1.piece < t_end;
        q0 = q1;
        q1 = q2;
        advance(q2);
        return more;
    };
    for (;;) {
        if (!step(ca, cc)) break;
        if (!step(cb, ca)) break;
        if (!step(cc, cb)) break;
    }
}

// The pieces of split tiles, one workgroup per tile and one thread per row
// (kTile blocks of at most 8 rows): y of a row = the sum of its partial
// sums in piece order, scaled as a whole tile's would be (deterministic:
// the same order on every call).  Every piece's partial sum is requested
// before the first is added, so the loads wait once, not once per piece.
template <int TILE> constexpr int reduce_threads() { return TILE * 8; }
template <bool Q4>
__global__ __launch_bounds__(reduce_threads<StreamGeo<Q4>::kTile>()) void group_reduce_kernel(
    const GroupItem* items, const uint32_t* tile_item, const float* partial, const float* scales, uint32_t pieces,
    uint32_t rows_total) {
    constexpr int kTile = StreamGeo<Q4>::kTile;
    const uint32_t tile = blockIdx.x;
    const uint32_t i = tile_item[tile];
    const GroupItem* it = items + i;
    const uint32_t blk0 = (tile - it->tile0) * kTile;
    const uint32_t nblk = it->nb - blk0 < uint32_t(kTile) ? it->nb - blk0 : uint32_t(kTile);
    const uint32_t R = it->R, row0 = it->row0;
    const uint32_t r = threadIdx.x;
    if (r >= nblk * R) return;
    const uint32_t g = blk0 * R + r;   // row of the linear
    float v[kMaxPieces];
#pragma unroll
    for (uint32_t p = 0; p < kMaxPieces; ++p) v[p] = p < pieces ? partial[size_t(p) * rows_total + row0 + g] : 0.0f;
    float acc = 0.0f;
#pragma unroll
    for (uint32_t p = 0; p < kMaxPieces; ++p)
        if (p < pieces) acc += v[p];
    float m = scales[i];
    if constexpr (Q4) m *= f16_bits_to_f32(it->bscale[g / R]);
    it->y[g] = acc * m;
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

struct GroupTotals {
    uint64_t nfrag = 0, ntiles = 0, nzb = 0;
    size_t x_lds = 0;      // largest x in LDS (16-byte aligned)
    uint32_t col_lds = 0;  // staged columns per Z workgroup (at least the Z slice)
    bool q4 = false;       // the items have 4-bit codes (else binary16 buckets)
    int tile = 0;          // row blocks per stream tile
    int ks = 0;            // K-steps per stream chunk
    uint64_t rows = 0;     // rows of all linears
    uint32_t min_chunks = 0xFFFFFFFFu;   // fewest chunks of any linear's tile
    uint32_t pieces = 1;   // pieces per tile (see split_pieces)
    uint32_t zslice = kZSlice;   // buckets per Z workgroup
};

// Tiles split into pieces when there are fewer tiles than stream waves (a
// decoder layer's few large tiles would leave most waves idle): about one
// unit per wave, at most kMaxPieces, and no more pieces than the chunks of
// the shortest tile, so that no piece is empty.
inline uint32_t split_pieces(const GroupTotals& t, int64_t nwaves) {
    if (t.ntiles == 0 || t.ntiles >= uint64_t(nwaves)) return 1;
    uint64_t p = uint64_t(nwaves) / t.ntiles;
    p = p < kMaxPieces ? p : kMaxPieces;
    p = p < t.min_chunks ? p : t.min_chunks;
    return p < 1 ? 1u : uint32_t(p);
}

// Stream tiles of a linear with nb row blocks, and the balancing cost of one
// (its chunks in units of a quarter chunk: binary16 K-steps, plus the fixed
// part); the same for every item of a group.
inline uint32_t tiles_of(const Shape& s, const GroupTotals& t) { return uint32_t((s.nb + t.tile - 1) / t.tile); }
inline uint64_t tile_cost(const Shape& s, const GroupTotals& t) {
    return uint64_t(s.Bg / 32) * 4 / uint64_t(t.ks) + kTileFixedCost;
}

// LDS for the columns of one Z workgroup: the expected run, zslice buckets
// x R*N/Bg columns per bucket, plus a quarter and the alignment pieces; the
// rare slice beyond it reads its columns from global memory.
inline uint32_t col_lds_of(const Shape& s, uint32_t zslice) {
    const uint64_t expect = (uint64_t(zslice) * uint64_t(s.R) * uint64_t(s.N) / uint64_t(s.Bg) + 7) / 8;
    uint64_t bytes = 16 * (expect + expect / 4 + uint64_t(s.R) + 16);
    bytes = bytes < kZSliceBytes ? kZSliceBytes : bytes;
    bytes = bytes > kColLds ? kColLds : bytes;
    return uint32_t(bytes);
}

inline uint32_t z_blocks(int64_t Bg, uint32_t zslice) { return uint32_t((Bg + zslice - 1) / zslice); }

// Every item: a uniform single-row sketch with R in {2, 4, 8}, all of one
// bucket format (binary16 buckets with Bg a multiple of 32, or 4-bit codes
// with Bg a multiple of 128), whose x (with a Z slice) fits group_z_kernel's
// LDS, with 16-byte aligned device pointers.
sketch_status check_items(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype, GroupTotals* t) {
    if (!items || count < 1 || count > SKETCH_GROUP_MAX_ITEMS) return SKETCH_EINVAL;
    if (x_dtype != SKETCH_F32 && x_dtype != SKETCH_BF16 && x_dtype != SKETCH_F16) return SKETCH_EINVAL;
    const size_t xb = x_dtype == SKETCH_F32 ? 4 : 2;
    uint64_t nzb_big = 0, nzb_small = 0;   // Z workgroups with slices of kZSlice and of the small size
    uint32_t cl_big = 0, cl_small = 0;
    for (int32_t i = 0; i < count; ++i) {
        const sketch_group_item& g = items[i];
        Shape s;
        const sketch_status rc = validate_params(g.p, &s);
        if (rc != SKETCH_OK) return rc;
        if (s.rows != 1 || s.boff) return SKETCH_EINVAL;
        if (i == 0) {
            t->q4 = s.bits == 4;
            t->tile = t->q4 ? StreamGeo<true>::kTile : StreamGeo<false>::kTile;
            t->ks = t->q4 ? StreamGeo<true>::kKS : StreamGeo<false>::kKS;
        } else if ((s.bits == 4) != t->q4) {
            return SKETCH_EINVAL;   // one bucket format per group
        }
        if (!(s.R == 2 || s.R == 4 || s.R == 8) || s.Bg % (t->q4 ? 128 : 32) != 0 || s.nb < 1) return SKETCH_EINVAL;
        const uint64_t row_bytes = t->q4 ? uint64_t(s.Bg) / 2 : uint64_t(s.Bg) * 2;
        if (uint64_t(s.nb) * row_bytes >= (uint64_t(1) << 32)) return SKETCH_EINVAL;   // 32-bit offsets
        const size_t need = ((size_t(s.N) * xb + 15) & ~size_t(15)) + kColLds;
        if (need > kZLds) return SKETCH_EINVAL;
        auto misaligned = [](const void* q) { return !q || (reinterpret_cast<uintptr_t>(q) & 15u); };
        if (misaligned(g.proj) || misaligned(g.tables) || misaligned(g.x) || misaligned(g.y)) return SKETCH_EINVAL;
        const size_t xl = (size_t(s.N) * xb + 15) & ~size_t(15);
        t->x_lds = xl > t->x_lds ? xl : t->x_lds;
        const uint32_t small = t->q4 ? kZSliceQ4Small : kZSlice16Small;
        const uint32_t cb = col_lds_of(s, kZSlice), cs = col_lds_of(s, small);
        cl_big = cb > cl_big ? cb : cl_big;
        cl_small = cs > cl_small ? cs : cl_small;
        nzb_big += z_blocks(s.Bg, kZSlice);
        nzb_small += z_blocks(s.Bg, small);
        t->nfrag += uint64_t(s.Bg / 32) * 64;
        t->ntiles += tiles_of(s, *t);
        t->rows += uint64_t(s.M);
        const uint32_t nc = uint32_t((s.Bg / 32 + t->ks - 1) / t->ks);
        t->min_chunks = nc < t->min_chunks ? nc : t->min_chunks;
    }
    if (t->nfrag >= (uint64_t(1) << 28) || t->ntiles >= (uint64_t(1) << 31) || t->rows >= (uint64_t(1) << 31))
        return SKETCH_EINVAL;
    t->pieces = split_pieces(*t, group_waves(t->q4));
    const bool small = nzb_big < kZSmallBelow;
    t->zslice = small ? (t->q4 ? kZSliceQ4Small : kZSlice16Small) : kZSlice;
    t->nzb = small ? nzb_small : nzb_big;
    t->col_lds = small ? cl_small : cl_big;
    return SKETCH_OK;
}

// Plan entries of the tiles' linears: only when tiles are split.
inline uint64_t tile_items(const GroupTotals& t) { return t.pieces > 1 ? t.ntiles : 0; }

// Workspace: the Z fragments, one scale per linear, and when tiles are
// split the partial sums [pieces][rows].
inline size_t group_ws_bytes(int32_t count, const GroupTotals& t) {
    return align256(size_t(t.nfrag) * 16) + align256(size_t(count) * 4) +
           (t.pieces > 1 ? align256(size_t(t.pieces) * size_t(t.rows) * 4) : 0);
}

}  // namespace
}  // namespace sketch

using namespace sketch;

extern "C" sketch_status sketch_group_bytes(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                            size_t* plan_bytes, size_t* workspace_bytes) {
    GroupTotals t;
    const sketch_status rc = check_items(items, count, x_dtype, &t);
    if (rc != SKETCH_OK) return rc;
    if (plan_bytes) *plan_bytes = plan_layout(count, group_waves(t.q4), t.nzb, tile_items(t)).total;
    if (workspace_bytes) *workspace_bytes = group_ws_bytes(count, t);
    return SKETCH_OK;
}

extern "C" sketch_status sketch_group_plan(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                           void* plan, size_t plan_bytes, void* stream) {
    GroupTotals t;
    const sketch_status rc = check_items(items, count, x_dtype, &t);
    if (rc != SKETCH_OK) return rc;
    if (!plan || (reinterpret_cast<uintptr_t>(plan) & 15u)) return SKETCH_EINVAL;
    const int64_t nwaves = group_waves(t.q4);
    if (nwaves > kMaxWaves) return SKETCH_EINVAL;
    const PlanLayout L = plan_layout(count, nwaves, t.nzb, tile_items(t));
    if (plan_bytes < L.total) return SKETCH_ESMALL;
    PlanWriter w(plan, static_cast<hipStream_t>(stream));
    const GroupHeader h{kGroupMagic,      uint32_t(count),    uint32_t(t.ntiles), uint32_t(nwaves),
                        uint32_t(t.nfrag), uint32_t(x_dtype), uint32_t(t.nzb),    uint32_t(t.tile),
                        t.q4 ? 4u : 16u,   t.pieces,          uint32_t(t.rows),   t.zslice};
    w.put_bytes(0, &h, sizeof(h));
    // The items, and the cost of the tile stream: a tile streams its chunks,
    // plus a fixed part for its outputs (tile_cost); each of its pieces
    // counts the same.
    const uint32_t P = t.pieces;
    uint32_t tile0 = 0, frag0 = 0, zb0 = 0, row0 = 0;
    uint64_t total_cost = 0;
    for (int32_t i = 0; i < count; ++i) {
        Shape s;
        (void)validate_params(items[i].p, &s);
        const ProjLayout PL = proj_layout(s.R, s.N, s.Bg);
        const char* pb = static_cast<const char*>(items[i].proj);
        GroupItem g;
        g.S = items[i].tables;
        g.x = items[i].x;
        g.y = items[i].y;
        g.hdr = reinterpret_cast<const ProjHeader*>(pb);
        g.off = reinterpret_cast<const uint32_t*>(pb + PL.off);
        g.cols = reinterpret_cast<const uint16_t*>(pb + PL.cols);
        g.bscale = t.q4 ? reinterpret_cast<const uint16_t*>(reinterpret_cast<const char*>(items[i].tables) +
                                                            q4_scales_offset(s))
                        : nullptr;
        g.N = uint32_t(s.N);
        g.R = uint32_t(s.R);
        g.Bg = uint32_t(s.Bg);
        g.seed = items[i].p->seed;
        g.nb = uint32_t(s.nb);
        g.tile0 = tile0;
        g.frag0 = frag0;
        g.zb0 = zb0;
        g.row0 = row0;
        g.pad = 0;
        w.put_bytes(L.items + sizeof(GroupItem) * size_t(i), &g, sizeof(g));
        const uint32_t nt = tiles_of(s, t);
        tile0 += nt;
        frag0 += uint32_t(s.Bg / 32) * 64;
        zb0 += z_blocks(s.Bg, t.zslice);
        row0 += uint32_t(s.M);
        total_cost += uint64_t(nt) * P * tile_cost(s, t);
    }
    // Units: tile * P + piece, in tile order.  Wave v starts at the first
    // unit whose cost prefix reaches v * total / nwaves; its first item is
    // recorded with it.
    const uint32_t nunits = uint32_t(t.ntiles) * P;
    uint32_t wave_tile[kMaxWaves + 1], wave_item[kMaxWaves];
    {
        uint32_t unit = 0, item = 0, done = 0, nu = 0;
        uint64_t cost = 0, cc = 0;
        auto enter = [&](uint32_t i) {
            Shape s;
            (void)validate_params(items[i].p, &s);
            nu = tiles_of(s, t) * P;
            cc = tile_cost(s, t);
        };
        enter(0);
        for (int64_t v = 0; v < nwaves; ++v) {
            const uint64_t target = uint64_t((__uint128_t(total_cost) * uint64_t(v)) / uint64_t(nwaves));
            while (cost < target && unit < nunits) {
                cost += cc;
                ++unit;
                if (++done == nu && item + 1 < uint32_t(count)) {
                    ++item;
                    done = 0;
                    enter(item);
                }
            }
            wave_tile[v] = unit;
            wave_item[v] = item;
        }
        wave_tile[nwaves] = nunits;
    }
    for (int64_t v = 0; v <= nwaves; ++v) w.put(L.wave_tile / 4 + size_t(v), wave_tile[v]);
    for (int64_t v = 0; v < nwaves; ++v) w.put(L.wave_item / 4 + size_t(v), wave_item[v]);
    size_t at = L.zb_item / 4;
    for (int32_t i = 0; i < count; ++i) {
        Shape s;
        (void)validate_params(items[i].p, &s);
        for (uint32_t b = 0, nb = z_blocks(s.Bg, t.zslice); b < nb; ++b) w.put(at++, uint32_t(i));
    }
    if (P > 1) {   // the linear of every tile, for the sum of the pieces
        at = L.tile_item / 4;
        for (int32_t i = 0; i < count; ++i) {
            Shape s;
            (void)validate_params(items[i].p, &s);
            for (uint32_t k = 0, nt = tiles_of(s, t); k < nt; ++k) w.put(at++, uint32_t(i));
        }
    }
    w.flush();
    if (w.failed) return SKETCH_EDEVICE;
    char* pb = static_cast<char*>(plan);
    group_prep_kernel<<<unsigned((t.nzb + 255) / 256), 256, 0, static_cast<hipStream_t>(stream)>>>(
        reinterpret_cast<const GroupItem*>(pb + L.items), reinterpret_cast<const uint32_t*>(pb + L.zb_item),
        reinterpret_cast<ZRec*>(pb + L.zrec), uint32_t(t.nzb), t.zslice);
    return launch_status();
}

extern "C" sketch_status sketch_matmul_group(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                             const void* plan, void* workspace, size_t workspace_bytes, void* stream) {
    GroupTotals t;
    const sketch_status rc = check_items(items, count, x_dtype, &t);
    if (rc != SKETCH_OK) return rc;
    if (!plan || (reinterpret_cast<uintptr_t>(plan) & 15u)) return SKETCH_EINVAL;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u)) return SKETCH_EINVAL;
    if (workspace_bytes < group_ws_bytes(count, t)) return SKETCH_ESMALL;
    const int64_t nwaves = group_waves(t.q4);
    const PlanLayout L = plan_layout(count, nwaves, t.nzb, tile_items(t));
    const char* pb = static_cast<const char*>(plan);
    const GroupItem* gi = reinterpret_cast<const GroupItem*>(pb + L.items);
    half8* frags = static_cast<half8*>(workspace);
    float* scales = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(size_t(t.nfrag) * 16));
    hipStream_t st = static_cast<hipStream_t>(stream);
    const ZRec* zr = reinterpret_cast<const ZRec*>(pb + L.zrec);
    const unsigned nzb = unsigned(t.nzb);
    const size_t zlds = t.x_lds + t.col_lds;
    // SLICE buckets per workgroup of THREADS threads, RPT rows per thread
    auto launch_z = [&](auto q4, auto slice, auto threads) {
        constexpr bool Q4 = decltype(q4)::value;
        constexpr int THREADS = decltype(threads)::value;
        constexpr int RPT = decltype(slice)::value * 8 / THREADS;
        switch (x_dtype) {
            case SKETCH_F32:
                group_z_kernel<SKETCH_F32, Q4, RPT, THREADS><<<nzb, THREADS, zlds, st>>>(zr, frags, scales, t.col_lds);
                break;
            case SKETCH_BF16:
                group_z_kernel<SKETCH_BF16, Q4, RPT, THREADS><<<nzb, THREADS, zlds, st>>>(zr, frags, scales, t.col_lds);
                break;
            default:
                group_z_kernel<SKETCH_F16, Q4, RPT, THREADS><<<nzb, THREADS, zlds, st>>>(zr, frags, scales, t.col_lds);
                break;
        }
    };
    using Q4T = std::true_type;
    using B16 = std::false_type;
    using I256 = std::integral_constant<int, 256>;
    using I512 = std::integral_constant<int, 512>;
    if (t.q4 && t.zslice == kZSlice)
        launch_z(Q4T{}, std::integral_constant<int, kZSlice>{}, I256{});
    else if (t.q4)
        launch_z(Q4T{}, std::integral_constant<int, kZSliceQ4Small>{}, I256{});
    else if (t.zslice == kZSlice)
        launch_z(B16{}, std::integral_constant<int, kZSlice>{}, I512{});
    else
        launch_z(B16{}, std::integral_constant<int, kZSlice16Small>{}, I512{});
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    StreamArgs a;
    a.items = gi;
    a.wave_tile = reinterpret_cast<const uint32_t*>(pb + L.wave_tile);
    a.wave_item = reinterpret_cast<const uint32_t*>(pb + L.wave_item);
    a.frags = frags;
    a.scales = scales;
    a.count = uint32_t(count);
    a.nwaves = uint32_t(nwaves);
    a.nfrag = uint32_t(t.nfrag);
    a.pieces = t.pieces;
    a.rows_total = uint32_t(t.rows);
    a.partial = t.pieces > 1 ? reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(size_t(t.nfrag) * 16) +
                                                        align256(size_t(count) * 4))
                             : nullptr;
    const unsigned grid = unsigned(nwaves / (kStreamThreads / 64));
    if (t.q4)
        group_stream_kernel<true><<<grid, kStreamThreads, (kStreamThreads / 64) * StreamGeo<true>::kSlot, st>>>(a);
    else
        group_stream_kernel<false><<<grid, kStreamThreads, (kStreamThreads / 64) * StreamGeo<false>::kSlot, st>>>(a);
    if (t.pieces == 1) return launch_status();
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    const uint32_t* ti = reinterpret_cast<const uint32_t*>(pb + L.tile_item);
    constexpr unsigned kRedQ4 = reduce_threads<StreamGeo<true>::kTile>();
    constexpr unsigned kRed16 = reduce_threads<StreamGeo<false>::kTile>();
    if (t.q4)
        group_reduce_kernel<true><<<unsigned(t.ntiles), kRedQ4, 0, st>>>(gi, ti, a.partial, scales, t.pieces,
                                                                         uint32_t(t.rows));
    else
        group_reduce_kernel<false><<<unsigned(t.ntiles), kRed16, 0, st>>>(gi, ti, a.partial, scales, t.pieces,
                                                                          uint32_t(t.rows));
    return launch_status();
}

// group.hip -- grouped decode product: many sketched linears, each with its
// own input vector and output, in two launches.
//
// "Resumen Técnico" › Metodología §4: W_hat = S * P^T, so each linear's
// product factorises as y[b*R + r] = sum_k S[b][k] * Z[r][k] with
// Z = P^T x (Resultados › Ablación: the matrix form equals the sequential
// one).  A decoder step multiplies several linears (each with its own x) by
// one token; launched one by one, each is far too small to keep HBM busy.
// Here the whole set is one stream of bucket tables:
//   * group_frag_kernel, one workgroup per linear: x into LDS, Z summed per
//     (row, bucket) segment of the projection's inverse map (ascending j),
//     the token's power-of-two scale from max |Z|, and Z written to the
//     workspace as binary16 hi + lo MFMA fragments (every product exact, the
//     same split as the single-linear product);
//   * group_stream_kernel: the tables of all linears form one sequence of
//     16-block tiles; every wave streams a contiguous, cost-balanced range of
//     it (planned on the host), crossing from one linear to the next without
//     a barrier.  A tile streams in chunks of 8 K-steps: 16 rows x 512
//     contiguous bytes into registers one chunk ahead (with the chunk's Z
//     fragments, which stay in L2), through the wave's LDS slot into the
//     MFMA operand pattern, 8 f16 MFMAs (Z as A, tables as B), and the
//     hi + lo sums of each output row are scaled back and stored.
#include <algorithm>
#include <cstring>

#include "common.h"

namespace sketch {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr uint32_t kGroupMagic = 0x50524753u;   // "SGRP"
constexpr int kFragThreads = 256;
constexpr int kStreamThreads = 256;             // 4 waves
constexpr int kTile = 16;                       // row blocks per tile (MFMA columns)
constexpr uint32_t kSlotBytes = 16 * 512;       // a wave's LDS slot: 16 rows x 256 buckets
constexpr size_t kFragLds = 152 * 1024;         // x + Z of one linear in group_frag_kernel
constexpr int64_t kMaxWaves = 8192;             // waves of the stream launch (2 x 4 per CU)
constexpr uint32_t kTileFixedCost = 4;          // per-tile overhead, in K-steps, for the balancing

// One linear of the group, as the kernels read it.
struct alignas(16) GroupItem {
    const uint16_t* S;      // tables [nb][Bg]
    const void* x;          // [N]
    float* y;               // [M]
    const ProjHeader* hdr;  // projection (checked by group_frag_kernel)
    const uint32_t* off;    // inverse map offsets [R*Bg + 1]
    const uint16_t* cols;   // inverse map columns [R*N]
    uint32_t N, R, Bg, seed;
    uint32_t nb, tile0;     // row blocks; first tile in the group's tile order
    uint32_t frag0, pad;    // first 16-byte fragment of this linear in the workspace
};
static_assert(sizeof(GroupItem) == 80, "plan layout");

struct alignas(16) GroupHeader {
    uint32_t magic, count, ntiles, nwaves;
    uint32_t nfrag, xdt, pad[2];
};

// Plan: header | items[count] | wave_tile[nwaves + 1] | wave_item[nwaves]
struct PlanLayout {
    size_t items, wave_tile, wave_item, total;
};
inline PlanLayout plan_layout(int64_t count, int64_t nwaves) {
    PlanLayout L;
    L.items = align256(sizeof(GroupHeader));
    L.wave_tile = align256(L.items + sizeof(GroupItem) * size_t(count));
    L.wave_item = align256(L.wave_tile + 4 * size_t(nwaves + 1));
    L.total = align256(L.wave_item + 4 * size_t(nwaves));
    return L;
}

int group_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu > 0 ? ncu : 256;
}

// Waves of the streaming launch: two 4-wave workgroups per CU.
inline int64_t group_waves() { return int64_t(2 * group_cus()) * (kStreamThreads / 64); }

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

// ---------------------------------------------------------------------------
// Z fragments of one linear (one workgroup per linear).
// frag[s*64 + kq*16 + c] = 8 buckets k = 32 s + 8 kq + 0..7 of column c,
// c = 2 rr + h: the hi (h = 0) or lo (h = 1) binary16 part of Z[rr][k] * su;
// columns of rows rr >= R are zero.
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(kFragThreads) void group_frag_kernel(const GroupItem* items, half8* frags, float* scales) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    __shared__ uint32_t wmax[kFragThreads / 64];
    const GroupItem it = items[blockIdx.x];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr uint32_t xb = XDT == SKETCH_F32 ? 4u : 2u;
    unsigned char* xl = lds;
    float* zl = reinterpret_cast<float*>(lds + ((size_t(it.N) * xb + 15) & ~size_t(15)));
    const bool ok = it.hdr->magic == kProjMagic && it.hdr->version == kProjVersion && it.hdr->R == it.R &&
                    it.hdr->N == it.N && it.hdr->Bg == it.Bg && it.hdr->seed == it.seed;
    // x -> LDS (raw bits)
    if constexpr (XDT == SKETCH_F32) {
        for (uint32_t e = tid; e < it.N; e += kFragThreads)
            reinterpret_cast<uint32_t*>(xl)[e] = static_cast<const uint32_t*>(it.x)[e];
    } else {
        for (uint32_t e = tid; e < it.N; e += kFragThreads)
            reinterpret_cast<uint16_t*>(xl)[e] = static_cast<const uint16_t*>(it.x)[e];
    }
    __syncthreads();
    // Z[r][k]: the columns of each segment in ascending j
    const uint32_t nz = it.R * it.Bg;
    uint32_t mx = 0;
    for (uint32_t sgi = tid; sgi < nz; sgi += kFragThreads) {
        float z = 0.0f;
        if (ok) {
            const uint32_t b = it.off[sgi], e = it.off[sgi + 1];
            for (uint32_t c = b; c < e; ++c) {
                uint32_t j = it.cols[c];
                j = j < it.N ? j : it.N - 1;
                z += XDT == SKETCH_F32   ? reinterpret_cast<const float*>(xl)[j]
                     : XDT == SKETCH_BF16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(xl)[j])
                                          : f16_bits_to_f32(reinterpret_cast<const uint16_t*>(xl)[j]);
            }
        } else {
            z = __builtin_nanf("");
        }
        zl[sgi] = z;
        const float m = __builtin_fabsf(z);
        const uint32_t mb = m <= 3.402823466e38f ? __float_as_uint(m) : 0x7F800000u;
        mx = mb > mx ? mb : mx;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t t = uint32_t(__shfl_xor(int(mx), o));
        mx = t > mx ? t : mx;
    }
    if (lane == 0) wmax[wave] = mx;
    __syncthreads();
    uint32_t mall = wmax[0];
#pragma unroll
    for (int w = 1; w < kFragThreads / 64; ++w) mall = wmax[w] > mall ? wmax[w] : mall;
    // power-of-two scale bringing max |Z| into [2^14, 2^15); none for a zero
    // or non-finite maximum, and at most 2^±120
    const float m = __uint_as_float(mall);
    int e = 0;
    if (m <= 3.402823466e38f && m > 0.0f) {
        e = 14 - ilogbf(m);
        e = e > 120 ? 120 : e < -120 ? -120 : e;
    }
    const float su = ldexpf(1.0f, e);
    if (tid == 0) scales[blockIdx.x] = ldexpf(1.0f, -e);
    // fragments
    const uint32_t nst = it.Bg / 32, nf = nst * 64;
    half8* fr = frags + it.frag0;
    for (uint32_t f = tid; f < nf; f += kFragThreads) {
        const uint32_t s = f >> 6, kq = (f >> 4) & 3, c = f & 15, rr = c >> 1, h = c & 1;
        half8 out = half8{};
        if (rr < it.R) {
            const float* zr = zl + rr * it.Bg + s * 32 + kq * 8;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float v = zr[i] * su;
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
// The tile stream.
// ---------------------------------------------------------------------------
struct StreamArgs {
    const GroupItem* items;
    const uint32_t* wave_tile;   // [nwaves + 1]
    const uint32_t* wave_item;   // [nwaves]
    const half8* frags;
    const float* scales;
    uint32_t count, nwaves;
};

__global__ __launch_bounds__(kStreamThreads) void group_stream_kernel(StreamArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // XCD-aware numbering: the workgroups of one XCD take consecutive wave
    // ranges, so each XCD's L2 holds the fragments of its own linears
    uint32_t bid = blockIdx.x;
    if ((gridDim.x & 7u) == 0) bid = (bid & 7u) * (gridDim.x >> 3) + (bid >> 3);
    const uint32_t gw = bid * (kStreamThreads / 64) + uint32_t(wave);
    if (gw >= a.nwaves) return;
    const uint32_t t_begin = a.wave_tile[gw], t_end = a.wave_tile[gw + 1];
    if (t_begin >= t_end) return;
    unsigned char* slot = lds + size_t(wave) * kSlotBytes;
    const uint32_t n = uint32_t(lane) & 15u, qd = uint32_t(lane) >> 4;

    // chunk cursor: (item, tile, chunk) with the item's geometry cached
    struct Cursor {
        uint32_t item, tile, c;
        GroupItem it;
    };
    auto load_item = [&](uint32_t i, GroupItem& it) { it = a.items[i < a.count ? i : a.count - 1]; };
    auto nchunks_of = [](const GroupItem& it) { return (it.Bg / 32 + 7) / 8; };
    auto advance = [&](Cursor& q) {
        if (++q.c >= nchunks_of(q.it)) {
            q.c = 0;
            ++q.tile;
            if (q.tile >= q.it.tile0 + (q.it.nb + kTile - 1) / kTile && q.item + 1 < a.count) {
                ++q.item;
                load_item(q.item, q.it);
            }
        }
    };
    // 8 x 16 bytes per lane: rows 2i + lane/32 of the tile, buckets
    // 256c + 8 (lane % 32) .. +8; past the end of a row or of the linear the
    // addresses are clamped (loaded, never used).  The chunk's 8 Z fragments
    // go out with it.
    auto load_chunk = [&](const Cursor& q, u32x4 (&v)[8], half8 (&f)[8]) {
        const GroupItem& it = q.it;
        const uint32_t lt = q.tile - it.tile0;
        uint32_t col = q.c * 256 + (uint32_t(lane) & 31) * 8;
        col = col + 8 <= it.Bg ? col : it.Bg - 8;
        const uint32_t nst = it.Bg / 32;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t row = lt * kTile + 2 * i + (uint32_t(lane) >> 5);
            row = row < it.nb ? row : it.nb - 1;
            v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(it.S + size_t(row) * it.Bg + col));
            uint32_t s = q.c * 8 + uint32_t(i);
            s = s < nst ? s : nst - 1;
            f[i] = a.frags[it.frag0 + s * 64 + uint32_t(lane)];
        }
    };

    Cursor cur;
    cur.item = a.wave_item[gw];
    load_item(cur.item, cur.it);
    cur.tile = t_begin;
    cur.c = 0;
    Cursor nxt = cur;
    u32x4 va[8], vb[8];
    half8 fa[8], fb[8];
    load_chunk(cur, va, fa);
    float4v acc = float4v{0.f, 0.f, 0.f, 0.f};

    auto do_chunk = [&](const Cursor& q, const u32x4 (&v)[8], const half8 (&f)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) *reinterpret_cast<u32x4*>(slot + i * 1024 + uint32_t(lane) * 16) = v[i];
        const unsigned char* sl = slot + n * 512 + qd * 16;
        const uint32_t nst = q.it.Bg / 32;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) {
            const half8 bv = *reinterpret_cast<const half8*>(sl + s8 * 64);
            if (q.c * 8 + uint32_t(s8) < nst)   // wave-uniform
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(f[s8], bv, acc, 0, 0, 0);
        }
        if (q.c + 1 == nchunks_of(q.it)) {
            // lane (n, qd): rows 2qd and 2qd + 1 (hi + lo columns) of block n
            const GroupItem& it = q.it;
            const uint32_t blk = (q.tile - it.tile0) * kTile + n, r0 = 2 * qd;
            if (blk < it.nb && r0 < it.R) {
                const float sd = a.scales[q.item];
                const float y0 = (acc[0] + acc[1]) * sd, y1 = (acc[2] + acc[3]) * sd;
                float* yp = it.y + size_t(blk) * it.R + r0;
                if (r0 + 1 < it.R)
                    __builtin_nontemporal_store(float2v{y0, y1}, reinterpret_cast<float2v*>(yp));
                else
                    *yp = y0;
            }
            acc = float4v{0.f, 0.f, 0.f, 0.f};
        }
    };

    // chunks in pairs: A holds the current chunk, B is filled with the next
    for (;;) {
        advance(nxt);
        const bool more = nxt.tile < t_end;
        if (more) load_chunk(nxt, vb, fb);
        do_chunk(cur, va, fa);
        if (!more) break;
        cur = nxt;
        advance(nxt);
        const bool more2 = nxt.tile < t_end;
        if (more2) load_chunk(nxt, va, fa);
        do_chunk(cur, vb, fb);
        if (!more2) break;
        cur = nxt;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

struct GroupTotals {
    uint64_t nfrag = 0, ntiles = 0;
    size_t frag_lds = 0;
};

// Every item: a uniform single-row binary16 sketch with R in {2, 4, 8} and
// Bg a multiple of 32, whose x (and its Z) fit group_frag_kernel's LDS, with
// 16-byte aligned device pointers.
sketch_status check_items(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype, GroupTotals* t) {
    if (!items || count < 1 || count > SKETCH_GROUP_MAX_ITEMS) return SKETCH_EINVAL;
    if (x_dtype != SKETCH_F32 && x_dtype != SKETCH_BF16 && x_dtype != SKETCH_F16) return SKETCH_EINVAL;
    const size_t xb = x_dtype == SKETCH_F32 ? 4 : 2;
    for (int32_t i = 0; i < count; ++i) {
        const sketch_group_item& g = items[i];
        Shape s;
        const sketch_status rc = validate_params(g.p, &s);
        if (rc != SKETCH_OK) return rc;
        if (s.rows != 1 || s.boff || s.bits != 16) return SKETCH_EINVAL;
        if (!(s.R == 2 || s.R == 4 || s.R == 8) || s.Bg % 32 != 0 || s.nb < 1) return SKETCH_EINVAL;
        const size_t need = ((size_t(s.N) * xb + 15) & ~size_t(15)) + size_t(s.R) * size_t(s.Bg) * 4;
        if (need > kFragLds) return SKETCH_EINVAL;
        auto misaligned = [](const void* q) { return !q || (reinterpret_cast<uintptr_t>(q) & 15u); };
        if (misaligned(g.proj) || misaligned(g.tables) || misaligned(g.x) || misaligned(g.y)) return SKETCH_EINVAL;
        t->frag_lds = need > t->frag_lds ? need : t->frag_lds;
        t->nfrag += uint64_t(s.Bg / 32) * 64;
        t->ntiles += uint64_t((s.nb + kTile - 1) / kTile);
    }
    if (t->nfrag >= (uint64_t(1) << 31) || t->ntiles >= (uint64_t(1) << 31)) return SKETCH_EINVAL;
    return SKETCH_OK;
}

inline size_t group_ws_bytes(int32_t count, const GroupTotals& t) {
    return align256(size_t(t.nfrag) * 16) + align256(size_t(count) * 4);
}

}  // namespace
}  // namespace sketch

using namespace sketch;

extern "C" sketch_status sketch_group_bytes(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                            size_t* plan_bytes, size_t* workspace_bytes) {
    GroupTotals t;
    const sketch_status rc = check_items(items, count, x_dtype, &t);
    if (rc != SKETCH_OK) return rc;
    if (plan_bytes) *plan_bytes = plan_layout(count, group_waves()).total;
    if (workspace_bytes) *workspace_bytes = group_ws_bytes(count, t);
    return SKETCH_OK;
}

extern "C" sketch_status sketch_group_plan(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                           void* plan, size_t plan_bytes, void* stream) {
    GroupTotals t;
    const sketch_status rc = check_items(items, count, x_dtype, &t);
    if (rc != SKETCH_OK) return rc;
    if (!plan || (reinterpret_cast<uintptr_t>(plan) & 15u)) return SKETCH_EINVAL;
    const int64_t nwaves = group_waves();
    if (nwaves > kMaxWaves) return SKETCH_EINVAL;
    const PlanLayout L = plan_layout(count, nwaves);
    if (plan_bytes < L.total) return SKETCH_ESMALL;
    PlanWriter w(plan, static_cast<hipStream_t>(stream));
    const GroupHeader h{kGroupMagic, uint32_t(count), uint32_t(t.ntiles), uint32_t(nwaves), uint32_t(t.nfrag),
                        uint32_t(x_dtype), {0, 0}};
    w.put_bytes(0, &h, sizeof(h));
    // The items, and the cost of the tile stream: a tile of a linear with Bg
    // buckets streams Bg / 32 K-steps, plus a fixed part for its outputs.
    uint32_t tile0 = 0, frag0 = 0;
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
        g.N = uint32_t(s.N);
        g.R = uint32_t(s.R);
        g.Bg = uint32_t(s.Bg);
        g.seed = items[i].p->seed;
        g.nb = uint32_t(s.nb);
        g.tile0 = tile0;
        g.frag0 = frag0;
        g.pad = 0;
        w.put_bytes(L.items + sizeof(GroupItem) * size_t(i), &g, sizeof(g));
        const uint32_t nt = uint32_t((s.nb + kTile - 1) / kTile);
        tile0 += nt;
        frag0 += uint32_t(s.Bg / 32) * 64;
        total_cost += uint64_t(nt) * uint64_t(s.Bg / 32 + kTileFixedCost);
    }
    // Wave v starts at the first tile whose cost prefix reaches
    // v * total / nwaves; its first item is recorded with it.
    uint32_t wave_tile[kMaxWaves + 1], wave_item[kMaxWaves];
    {
        uint32_t tile = 0, item = 0, done = 0, nt = 0;
        uint64_t cost = 0, cc = 0;
        auto enter = [&](uint32_t i) {
            Shape s;
            (void)validate_params(items[i].p, &s);
            nt = uint32_t((s.nb + kTile - 1) / kTile);
            cc = uint64_t(s.Bg / 32 + kTileFixedCost);
        };
        enter(0);
        for (int64_t v = 0; v < nwaves; ++v) {
            const uint64_t target = uint64_t((__uint128_t(total_cost) * uint64_t(v)) / uint64_t(nwaves));
            while (cost < target && tile < t.ntiles) {
                cost += cc;
                ++tile;
                if (++done == nt && item + 1 < uint32_t(count)) {
                    ++item;
                    done = 0;
                    enter(item);
                }
            }
            wave_tile[v] = tile;
            wave_item[v] = item;
        }
        wave_tile[nwaves] = uint32_t(t.ntiles);
    }
    for (int64_t v = 0; v <= nwaves; ++v) w.put(L.wave_tile / 4 + size_t(v), wave_tile[v]);
    for (int64_t v = 0; v < nwaves; ++v) w.put(L.wave_item / 4 + size_t(v), wave_item[v]);
    w.flush();
    return w.failed ? SKETCH_EDEVICE : SKETCH_OK;
}

extern "C" sketch_status sketch_matmul_group(const sketch_group_item* items, int32_t count, sketch_dtype x_dtype,
                                             const void* plan, void* workspace, size_t workspace_bytes, void* stream) {
    GroupTotals t;
    const sketch_status rc = check_items(items, count, x_dtype, &t);
    if (rc != SKETCH_OK) return rc;
    if (!plan || (reinterpret_cast<uintptr_t>(plan) & 15u)) return SKETCH_EINVAL;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 15u)) return SKETCH_EINVAL;
    if (workspace_bytes < group_ws_bytes(count, t)) return SKETCH_ESMALL;
    const int64_t nwaves = group_waves();
    const PlanLayout L = plan_layout(count, nwaves);
    const char* pb = static_cast<const char*>(plan);
    const GroupItem* gi = reinterpret_cast<const GroupItem*>(pb + L.items);
    half8* frags = static_cast<half8*>(workspace);
    float* scales = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(size_t(t.nfrag) * 16));
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (x_dtype) {
        case SKETCH_F32: group_frag_kernel<SKETCH_F32><<<unsigned(count), kFragThreads, t.frag_lds, st>>>(gi, frags, scales); break;
        case SKETCH_BF16: group_frag_kernel<SKETCH_BF16><<<unsigned(count), kFragThreads, t.frag_lds, st>>>(gi, frags, scales); break;
        case SKETCH_F16: group_frag_kernel<SKETCH_F16><<<unsigned(count), kFragThreads, t.frag_lds, st>>>(gi, frags, scales); break;
    }
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    StreamArgs a;
    a.items = gi;
    a.wave_tile = reinterpret_cast<const uint32_t*>(pb + L.wave_tile);
    a.wave_item = reinterpret_cast<const uint32_t*>(pb + L.wave_item);
    a.frags = frags;
    a.scales = scales;
    a.count = uint32_t(count);
    a.nwaves = uint32_t(nwaves);
    group_stream_kernel<<<unsigned(nwaves / (kStreamThreads / 64)), kStreamThreads,
                          (kStreamThreads / 64) * kSlotBytes, st>>>(a);
    return launch_status();
}

// encode.hip -- sketch compression on gfx950.
//
// "Resumen Técnico" › Metodología §1 (AbsMaxMin sketch): a bucket keeps the
// colliding weight of minimum absolute value.  Metodología §2: importance
// scales the choice (key = |w| * imp[j], one binary32 multiply).
// Metodología §4: selection and update are fused into one kernel, a MIN
// reduction through the projection P.
//
// Design (one workgroup per row block, persistent over blocks):
//   * The block's Bg buckets live in LDS as packed 64-bit words
//       word = key_bits << 32 | tie
//     where key_bits is the binary32 pattern of the non-negative key (its
//     unsigned order is the numeric order) and tie = l for AbsMin (LDS atomic
//     min: smaller key, then smaller l) or ~l for AbsMax (LDS atomic max:
//     larger key, then smaller l).  The result is independent of the order
//     in which lanes arrive, so the encode is deterministic.
//   * W is streamed once with 16-byte loads (8 bf16/fp16 or 2x4 fp32 per
//     chunk); the bucket of each position comes from the projection's
//     forward map (16-bit, shared by every block, cache-resident), so no hash
//     is recomputed per weight.
//   * After a barrier, each bucket's winner index is unpacked, the winning
//     weight is read back -- from the LDS copy of the block made while it
//     streamed by (when table and block fit), else from memory -- and
//     rounded to binary16; empty buckets store +0.  16-bit weights of
//     blocks of at most 2^17 weights carry their bits in the packed word
//     instead (31-bit key, 17-bit tie, 16-bit value), so neither is needed.
//   * For 16-bit weights of the single-row sketches the words are built with
//     about seven VALU instructions per weight (widening, one multiply, the
//     word halves by shift-or and alignbit, the slot address by one
//     v_mad_u32_u16) and the range check is one packed 16-bit max per two
//     weights; the general path takes about eleven.
//   * Weight range (NaN/Inf, |w| >= 65520) and importance validity are
//     checked on the fly and reported through the status word.
//   * Multi-row sketch (Metodología §1, several hash functions with a sketch
//     row each): the projection holds one forward map per row, with indices
//     into that row's own segment of the block's buckets, so a weight makes
//     one update per row into the same LDS table; everything else is the
//     single-row kernel.
//   * Importance-aware allocation (Metodología §2, more buckets for more
//     important rows): block b owns Bg_b buckets at its own table offset;
//     the projection holds the 32-bit hash H[l] of every local index and the
//     bucket is umulhi(H[l], Bg_b), one multiply per weight.
//   * 4-bit buckets (Resultados: 0.5 bpw with 4-bit quantization): the same
//     reduction over Bg = R*N*bpw/4 buckets; the output phase takes the
//     block's largest |winner|, the binary16 scale s = f16(max / 7) and packs
//     q = clamp(rint(w / s), -7, 7) two per byte (float32 divisions rounded
//     to nearest).
#include <mutex>

#include "common.h"

namespace sketch {
namespace {

// Status word of sketch_encode calls made without one of the caller's
// (status_dev == NULL): one per device, cleared, written and read back by
// the call itself, which then waits for its stream.  A process-wide lock
// keeps two such calls from sharing it at once.
__device__ __attribute__((aligned(16))) int32_t g_sync_status[4];

__global__ void clear_status_kernel(int32_t* w) {
    if (threadIdx.x == 0) *w = 0;
}

constexpr int kEncThreads = 512;   // 8 waves; two or three workgroups per CU (4 or 6 waves per SIMD)
constexpr int kRowGroup = 4;  // rows whose chunks are in flight together per thread
constexpr size_t kStashMax = 80 * 1024;  // table + stashed block per workgroup (two workgroups per CU: 160 KiB)

struct EncArgs {
    const void* W;
    const float* imp;
    const uint16_t* idx;
    const ProjHeader* hdr;
    uint16_t* S;
    int32_t* status;
    int64_t N, nb;
    uint32_t R, Bg, seed;
    uint32_t rows;   // sketch rows (forward maps idx[rho * R * N + l])
    const uint32_t* boff;  // allocation: table offsets [nb + 1]
    uint32_t bg_max;       // allocation: largest block count (LDS table size)
    uint64_t total;        // allocation: uniform budget nb * Bg the tables were sized for
    uint16_t* scales;      // 4-bit buckets: per-block binary16 scales
    uint32_t cpr;    // 8-element chunks per row (vector path)
    uint32_t nchunk; // chunks per block
};

template <int RULE>
__device__ inline void bucket_update(uint64_t* tab, uint32_t k, float key, uint32_t l) {
    uint64_t word = (uint64_t(__float_as_uint(key)) << 32) | uint64_t(RULE == SKETCH_ABSMIN ? l : ~l);
    if constexpr (RULE == SKETCH_ABSMIN)
        atomicMin(reinterpret_cast<unsigned long long*>(&tab[k]), (unsigned long long)word);
    else
        atomicMax(reinterpret_cast<unsigned long long*>(&tab[k]), (unsigned long long)word);
}

// Packed word of a weight whose 16-bit source bits ride along (blocks of at
// most 2^17 weights): key bits (31: the key is non-negative) << 33 | tie (17
// bits) << 16 | the weight's bfloat16/binary16 bits.  The order is that of
// bucket_update's words (key, then tie; ties are unique), and the winner's
// value comes out of its word, so no copy of the block is needed.
constexpr uint32_t kPackedMaxL = 1u << 17;
template <int RULE>
__device__ inline void bucket_update_packed(uint64_t* tab, uint32_t k, float key, uint32_t l, uint32_t bits16) {
    const uint32_t tie = RULE == SKETCH_ABSMIN ? l : (~l & (kPackedMaxL - 1));
    const uint64_t word = (uint64_t(__float_as_uint(key)) << 33) | (uint64_t(tie) << 16) | uint64_t(bits16);
    if constexpr (RULE == SKETCH_ABSMIN)
        atomicMin(reinterpret_cast<unsigned long long*>(&tab[k]), (unsigned long long)word);
    else
        atomicMax(reinterpret_cast<unsigned long long*>(&tab[k]), (unsigned long long)word);
}

// LDS byte address base + 8 * (16-bit half HI of packed), one v_mad_u32_u16.
template <int HI>
__device__ inline uint32_t lds_slot(uint32_t packed, uint32_t eight, uint32_t base) {
    uint32_t d;
    if (HI)
        asm("v_mad_u32_u16 %0, %1, %2, %3 op_sel:[1,0,0,0]" : "=v"(d) : "v"(packed), "s"(eight), "v"(base));
    else
        asm("v_mad_u32_u16 %0, %1, %2, %3" : "=v"(d) : "v"(packed), "s"(eight), "v"(base));
    return d;
}

typedef __attribute__((address_space(3))) unsigned long long lds_u64;
template <int RULE>
__device__ inline void lds_atomic_word(uint32_t addr, uint32_t lo, uint32_t hi) {
    const unsigned long long w = (uint64_t(hi) << 32) | lo;
    lds_u64* p = reinterpret_cast<lds_u64*>(static_cast<uintptr_t>(addr));
    if constexpr (RULE == SKETCH_ABSMIN)
        __hip_atomic_fetch_min(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    else
        __hip_atomic_fetch_max(p, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

enum { kEncUniform = 0, kEncRows = 1, kEncAlloc = 2, kEncQ4 = 3 };
// Where the output phase finds a winner's value: read again from memory, in
// the LDS copy of the block, or in the packed word itself.
enum { kWinMemory = 0, kWinStash = 1, kWinPacked = 2 };

template <int MODE>
__device__ inline bool header_ok(const ProjHeader* h, const EncArgs& a) {
    if constexpr (MODE == kEncAlloc)
        return h->magic == kProjMagicHash && h->version == kProjVersion && h->R == a.R && h->N == uint32_t(a.N) &&
               h->seed == a.seed;
    const bool magic = MODE == kEncRows ? (h->magic == kProjMagicRows && h->pad[0] == a.rows) : h->magic == kProjMagic;
    // (4-bit buckets use the binary16 sketch's projection for their bucket count)
    return magic && h->version == kProjVersion && h->R == a.R && h->N == uint32_t(a.N) && h->Bg == a.Bg &&
           h->seed == a.seed;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 8 consecutive elements of one row, widened to float.  W is read once:
// non-temporal loads keep it from displacing the cached forward map.
template <int WDT>
__device__ inline void load8(const void* W, int64_t e0, float (&f)[8]) {
    if constexpr (WDT == SKETCH_F32) {
        const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(W) + e0);
        f32x4 a = __builtin_nontemporal_load(p), b = __builtin_nontemporal_load(p + 1);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(W) + e0);
        u32x4 v = __builtin_nontemporal_load(p);
        uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if constexpr (WDT == SKETCH_BF16) {
                f[2 * i] = __uint_as_float(u[i] << 16);
                f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
            } else {
                f[2 * i] = f16_bits_to_f32(u[i] & 0xFFFFu);
                f[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
            }
        }
    }
}

// Range check of 8 widened weights: NaN, Inf or |w| >= 65520 (binary16 overflow).
__device__ inline bool out_of_range8(const float (&f)[8]) {
    float m = fmaxf(fmaxf(__builtin_fabsf(f[0]), __builtin_fabsf(f[1])), __builtin_fabsf(f[2]));
    m = fmaxf(fmaxf(m, __builtin_fabsf(f[3])), __builtin_fabsf(f[4]));
    m = fmaxf(fmaxf(m, __builtin_fabsf(f[5])), __builtin_fabsf(f[6]));
    m = fmaxf(m, __builtin_fabsf(f[7]));
    // fmaxf drops NaN operands, so NaN is caught by the unordered self-compare
    bool nan = false;
#pragma unroll
    for (int e = 0; e < 8; ++e) nan |= f[e] != f[e];
    return nan | !(m < 65520.0f);
}

// WIN == kWinStash: the block's weights are also written to LDS as they
// stream by, so the winners are read back from LDS instead of a second trip
// to memory (blocks up to 160 KiB with the table).  WIN == kWinPacked
// (bfloat16/binary16 weights, single-row uniform or 4-bit sketches, blocks
// of at most 2^17 weights): the packed words carry the weights' bits.  MODE: kEncUniform, kEncRows (a.rows
// forward maps; otherwise the extra-row loops compile out) or kEncAlloc
// (per-block counts and offsets, bucket = umulhi(H[l], Bg_b)).
// The uniform AbsMin sketch with packed words fits 80 registers without
// spilling, so three of its workgroups (six waves per SIMD) share a CU; every
// other variant needs more registers and runs at two.
template <int RULE, int WIN, int MODE>
constexpr int enc_waves_per_eu() {
    return WIN == kWinPacked && RULE == SKETCH_ABSMIN && MODE == kEncUniform ? 6 : 4;
}

template <int WDT, int RULE, bool VEC, int WIN, int MODE>
__global__ __launch_bounds__(kEncThreads) __attribute__((amdgpu_waves_per_eu(enc_waves_per_eu<RULE, WIN, MODE>())))
void encode_kernel(EncArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint64_t tab[];
    __shared__ float wave_max[kEncThreads / 64];   // 4-bit buckets: per-wave largest |winner|
    constexpr uint32_t ES = WDT == SKETCH_F32 ? 4 : 2;
    const int tid = threadIdx.x;
    constexpr uint64_t kIdent = RULE == SKETCH_ABSMIN ? ~uint64_t(0) : uint64_t(0);
    static_assert(WIN != kWinPacked || (VEC && WDT != SKETCH_F32 && (MODE == kEncUniform || MODE == kEncQ4)),
                  "packed words: 16-bit weights of single-row uniform or 4-bit sketches");
    constexpr bool STASH = WIN == kWinStash;
    // stashed block (STASH only), 16-byte aligned after the table
    const uint32_t tabn = MODE == kEncAlloc ? a.bg_max : a.Bg;   // LDS table entries
    unsigned char* wst = reinterpret_cast<unsigned char*>(tab) + ((size_t(tabn) * sizeof(uint64_t) + 15) & ~size_t(15));

    const uint32_t rows = MODE == kEncRows ? a.rows : 1u;
    if (!header_ok<MODE>(a.hdr, a)) {
        if (tid == 0 && blockIdx.x == 0) atomicOr(a.status, SKETCH_FLAG_PROJECTION);
        return;
    }

    const int64_t L = int64_t(a.R) * a.N;
    bool bad_w = false, bad_imp = false;
    u16x2 rmax = {0, 0};   // largest |w| bits of the 16-bit weights seen

    // Vector path work split: a thread owns 8-column chunks and walks the
    // rows of the block for each, so its importance values are loaded (and
    // validated) once per chunk, not once per weight.  With fewer chunks per
    // row than threads, several threads share a chunk column and split the
    // rows (row stride rs).
    const uint32_t cpr = a.cpr > 0 ? a.cpr : 1;
    const uint32_t T = kEncThreads;
    uint32_t cc0, cstep, r0, rs;
    if (cpr >= T) {
        cc0 = tid; cstep = T; r0 = 0; rs = 1;
    } else {
        rs = T / cpr;
        cc0 = tid % cpr; cstep = cpr; r0 = tid / cpr;
        if (r0 >= rs) r0 = a.R;  // idle thread
    }

    // The table starts cleared; the output phase resets every bucket it
    // reads, so each block needs only the two barriers of the loop (the same
    // sequence for every wave, whatever share of the work its lanes own).
    for (uint32_t q = tid; q < tabn; q += kEncThreads) tab[q] = kIdent;
    __syncthreads();

    constexpr int RG = ES == 4 ? kRowGroup / 2 : kRowGroup;
    bool bad_alloc = false;
    for (int64_t b = blockIdx.x; b < a.nb; b += gridDim.x) {
        const int64_t wbase = b * L;
        // this block's buckets: Bg at b * Bg, or Bg_b at its allocated offset
        uint32_t boff0 = uint32_t(b) * a.Bg, bgb = a.Bg;
        if constexpr (MODE == kEncAlloc) {
            if (!alloc_block(a.boff, b, a.bg_max, a.total, boff0, bgb)) {   // uniform over the workgroup
                bad_alloc = true;
                continue;
            }
        }
        if constexpr (VEC) {
            for (uint32_t cc = cc0; cc < cpr; cc += cstep) {
                // One group = rows rg, rg+rs, ... of chunk column cc.  Its loads
                // are issued unconditionally (rows past R re-read row 0 and are
                // then skipped), so the group is in flight at once and the
                // wait counters stay exact.
                // uniform block base + 32-bit per-lane offsets (scalar-base addressing)
                const unsigned char* wblk = static_cast<const unsigned char*>(a.W) + size_t(wbase) * ES;
                const unsigned char* iblk = reinterpret_cast<const unsigned char*>(a.idx);
                float im[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};   // |importance| of this column chunk
                for (uint32_t rg = r0; rg < a.R; rg += RG * rs) {
                    u32x4 wv[RG][ES / 2], kv[RG], kh[RG];
#pragma unroll
                    for (int u = 0; u < RG; ++u) {
                        uint32_t r = rg + u * rs;
                        r = r < a.R ? r : 0;
                        const uint32_t l0 = r * uint32_t(a.N) + cc * 8;
#pragma unroll
                        for (uint32_t h = 0; h < ES / 2; ++h)
                            wv[u][h] = __builtin_nontemporal_load(
                                reinterpret_cast<const u32x4*>(wblk + (l0 * ES + 16 * h)));
                        if constexpr (MODE == kEncAlloc) {   // 8 hashes: two 16-byte slices
                            kv[u] = *reinterpret_cast<const u32x4*>(iblk + size_t(l0) * 4u);
                            kh[u] = *reinterpret_cast<const u32x4*>(iblk + size_t(l0) * 4u + 16u);
                        } else {
                            kv[u] = *reinterpret_cast<const u32x4*>(iblk + l0 * 2u);
                            // multi-row: the second sketch row's slice goes out
                            // with the group too (a load in the update loop
                            // would make every update wait for it)
                            if constexpr (MODE == kEncRows)
                                kh[u] = *reinterpret_cast<const u32x4*>(iblk + (size_t(L) + l0) * 2u);
                        }
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    if (rg == r0) {
                        if (a.imp) {
                            const f32x4* ip = reinterpret_cast<const f32x4*>(a.imp + cc * 8);
                            const f32x4 i0 = ip[0], i1 = ip[1];
                            const float iv[8] = {i0.x, i0.y, i0.z, i0.w, i1.x, i1.y, i1.z, i1.w};
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                bad_imp |= !(iv[e] >= 0.0f && iv[e] <= 3.402823466e38f);
                                im[e] = __builtin_fabsf(iv[e]);
                            }
                        }
                    }
#pragma unroll
                    for (int u = 0; u < RG; ++u) {
                        const uint32_t r = rg + u * rs;
                        if (r >= a.R) continue;
                        const uint32_t l0 = r * uint32_t(a.N) + cc * 8;
                        if constexpr (STASH) {
#pragma unroll
                            for (uint32_t h = 0; h < ES / 2; ++h)
                                *reinterpret_cast<u32x4*>(wst + size_t(l0) * ES + 16 * h) = wv[u][h];
                        }
                        float w[8];
                        if constexpr (WDT == SKETCH_F32) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) w[e] = __uint_as_float(wv[u][e >> 2][e & 3]);
                        } else {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                if constexpr (WDT == SKETCH_BF16) {
                                    w[2 * i] = __uint_as_float(wv[u][0][i] << 16);
                                    w[2 * i + 1] = __uint_as_float(wv[u][0][i] & 0xFFFF0000u);
                                } else {
                                    w[2 * i] = f16_bits_to_f32(wv[u][0][i] & 0xFFFFu);
                                    w[2 * i + 1] = f16_bits_to_f32(wv[u][0][i] >> 16);
                                }
                            }
                        }
                        constexpr bool FAST16 = WDT != SKETCH_F32 && (MODE == kEncUniform || MODE == kEncQ4);
                        if constexpr (FAST16) {
                            // 16-bit weights of the single-row sketches: per weight one
                            // widening, one multiply, the word halves and the slot address
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                rmax = __builtin_elementwise_max(rmax, __builtin_bit_cast(u16x2, wv[u][0][i] & 0x7FFF7FFFu));
                            const uint32_t tb = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(tab));
                            const uint32_t eight = __builtin_amdgcn_readfirstlane(8u);
                            if constexpr (WIN == kWinPacked) {
                                const uint32_t base = RULE == SKETCH_ABSMIN ? l0 : (~l0 & (kPackedMaxL - 1));
                                const uint32_t hi_tie = base >> 16;
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const uint32_t d = wv[u][0][e >> 1];
                                    const uint32_t wb = (e & 1) ? (d & 0xFFFF0000u) : (d << 16);
                                    const float wf = WDT == SKETCH_BF16 ? __uint_as_float(wb)
                                                                        : f16_bits_to_f32((e & 1) ? d >> 16 : d & 0xFFFFu);
                                    const float key = __builtin_fabsf(wf) * im[e];
                                    const uint32_t hi = (__float_as_uint(key) << 1) | hi_tie;
                                    const uint32_t t = RULE == SKETCH_ABSMIN ? base + uint32_t(e) : base - uint32_t(e);
                                    const uint32_t lo = __builtin_amdgcn_alignbit(t, (e & 1) ? d : (d << 16), 16);
                                    const uint32_t addr = (e & 1) ? lds_slot<1>(kv[u][e >> 1], eight, tb)
                                                                  : lds_slot<0>(kv[u][e >> 1], eight, tb);
                                    lds_atomic_word<RULE>(addr, lo, hi);
                                }
                            } else {
                                const uint32_t base = RULE == SKETCH_ABSMIN ? l0 : ~l0;
#pragma unroll
                                for (int e = 0; e < 8; ++e) {
                                    const uint32_t d = wv[u][0][e >> 1];
                                    const float wf = WDT == SKETCH_BF16
                                                         ? __uint_as_float((e & 1) ? (d & 0xFFFF0000u) : (d << 16))
                                                         : f16_bits_to_f32((e & 1) ? d >> 16 : d & 0xFFFFu);
                                    const float key = __builtin_fabsf(wf) * im[e];
                                    const uint32_t lo = RULE == SKETCH_ABSMIN ? base + uint32_t(e) : base - uint32_t(e);
                                    const uint32_t addr = (e & 1) ? lds_slot<1>(kv[u][e >> 1], eight, tb)
                                                                  : lds_slot<0>(kv[u][e >> 1], eight, tb);
                                    lds_atomic_word<RULE>(addr, lo, __float_as_uint(key));
                                }
                            }
                            continue;
                        }
                        bad_w |= out_of_range8(w);
                        uint32_t ks[8];
                        if constexpr (MODE == kEncAlloc) {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                ks[e] = __umulhi(kv[u][e], bgb);
                                ks[4 + e] = __umulhi(kh[u][e], bgb);
                            }
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) ks[e] = (kv[u][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu;
                        }
                        if constexpr (WIN == kWinPacked) {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                bucket_update_packed<RULE>(tab, ks[e], __builtin_fabsf(w[e]) * im[e], l0 | uint32_t(e),
                                                           (wv[u][0][e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                bucket_update<RULE>(tab, ks[e], __builtin_fabsf(w[e]) * im[e], l0 | uint32_t(e));
                        }
                        for (uint32_t rho = 1; rho < rows; ++rho) {
                            const u32x4 kr = (MODE == kEncRows && rho == 1)
                                                 ? kh[u]
                                                 : *reinterpret_cast<const u32x4*>(iblk + (size_t(rho) * size_t(L) + l0) * 2u);
                            const uint32_t kq[8] = {kr.x & 0xFFFFu, kr.x >> 16, kr.y & 0xFFFFu, kr.y >> 16,
                                                    kr.z & 0xFFFFu, kr.z >> 16, kr.w & 0xFFFFu, kr.w >> 16};
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                bucket_update<RULE>(tab, kq[e], __builtin_fabsf(w[e]) * im[e], l0 | uint32_t(e));
                        }
                    }
                }
            }
        } else {
            for (int64_t l = tid; l < L; l += kEncThreads) {
                const int64_t j = l % a.N;
                float f = load_elem<WDT>(a.W, wbase + l);
                float im = a.imp ? a.imp[j] : 1.0f;
                float aw = __builtin_fabsf(f);
                bad_w |= !(aw < 65520.0f);
                bad_imp |= !(im >= 0.0f && im <= 3.402823466e38f);
                if constexpr (MODE == kEncAlloc)
                    bucket_update<RULE>(tab, __umulhi(reinterpret_cast<const uint32_t*>(a.idx)[l], bgb),
                                        aw * __builtin_fabsf(im), uint32_t(l));
                else
                    for (uint32_t rho = 0; rho < rows; ++rho)
                        bucket_update<RULE>(tab, a.idx[int64_t(rho) * L + l], aw * __builtin_fabsf(im), uint32_t(l));
            }
        }
        __syncthreads();

        // the winning weight of a packed word, from the stash or from memory
        auto winner = [&](uint64_t word) -> float {
            if constexpr (WIN == kWinPacked)
                return WDT == SKETCH_BF16 ? bf16_bits_to_f32(uint32_t(word) & 0xFFFFu)
                                          : f16_bits_to_f32(uint32_t(word) & 0xFFFFu);
            uint32_t l = uint32_t(word);
            if constexpr (RULE == SKETCH_ABSMAX) l = ~l;
            if constexpr (STASH) {
                if constexpr (WDT == SKETCH_F32)
                    return reinterpret_cast<const float*>(wst)[l];
                else if constexpr (WDT == SKETCH_BF16)
                    return bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(wst)[l]);
                else
                    return f16_bits_to_f32(reinterpret_cast<const uint16_t*>(wst)[l]);
            } else {
                return load_elem<WDT>(a.W, wbase + l);
            }
        };
        if constexpr (MODE == kEncQ4) {
            // block scale: the largest |winner| over the block (waves, then LDS)
            float m = 0.0f;
            for (uint32_t q = tid; q < a.Bg; q += kEncThreads) {
                const uint64_t word = tab[q];
                if (word != kIdent) m = fmaxf(m, __builtin_fabsf(winner(word)));
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
            if ((tid & 63) == 0) wave_max[tid >> 6] = m;
            __syncthreads();
            float amax = wave_max[0];
#pragma unroll
            for (int w = 1; w < kEncThreads / 64; ++w) amax = fmaxf(amax, wave_max[w]);
            const uint16_t s16 = f32_to_f16_bits(__fdiv_rn(amax, 7.0f));
            const float sc = f16_bits_to_f32(s16);
            uint8_t* Tb = reinterpret_cast<uint8_t*>(a.S) + b * int64_t(a.Bg / 2);
            for (uint32_t k = tid; k < a.Bg / 2; k += kEncThreads) {
                uint32_t byte = 0;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const uint32_t q = 2 * k + h;
                    const uint64_t word = tab[q];
                    tab[q] = kIdent;
                    int code = 0;
                    if (word != kIdent && sc > 0.0f) {
                        const float v = rintf(__fdiv_rn(winner(word), sc));
                        code = int(fminf(fmaxf(v, -7.0f), 7.0f));
                    }
                    byte |= uint32_t(code & 0xF) << (4 * h);
                }
                Tb[k] = uint8_t(byte);
            }
            if (tid == 0) a.scales[b] = s16;
        } else {
            uint16_t* Sb = a.S + boff0;
            for (uint32_t q = tid; q < bgb; q += kEncThreads) {
                const uint64_t word = tab[q];
                tab[q] = kIdent;
                Sb[q] = word != kIdent ? f32_to_f16_bits(winner(word)) : uint16_t(0);
            }
        }
        __syncthreads();
    }
    if constexpr (WDT != SKETCH_F32) {
        // bfloat16: |w| >= 65520 is |bits| >= 0x4780 (65536; nothing lies between);
        // binary16: only infinities and NaN (>= 0x7C00) reach 65520
        const uint32_t lim = WDT == SKETCH_BF16 ? 0x4780u : 0x7C00u;
        bad_w |= uint32_t(rmax.x) >= lim || uint32_t(rmax.y) >= lim;
    }
    int32_t flags = (bad_w ? SKETCH_FLAG_WEIGHT_RANGE : 0) | (bad_imp ? SKETCH_FLAG_IMPORTANCE : 0) |
                    (bad_alloc ? SKETCH_FLAG_ALLOCATION : 0);
    if (flags) atomicOr(a.status, flags);
}

template <int WDT, int RULE, int MODE>
sketch_status launch_typed(const EncArgs& a, bool vec, hipStream_t st) {
    const size_t es = WDT == SKETCH_F32 ? 4 : 2;
    const size_t tab_bytes = size_t(MODE == kEncAlloc ? a.bg_max : a.Bg) * sizeof(uint64_t);
    const size_t stash_bytes = ((tab_bytes + 15) & ~size_t(15)) + size_t(a.R) * size_t(a.N) * es;
    // 16-bit weights of blocks up to 2^17 weights carry their bits in the
    // packed words (the table alone, two or three workgroups per CU; measured a little
    // faster than the LDS copy of the block even where that fits: 11.1 vs
    // 11.6 us for the 4096x4096 weight in row blocks of 8).  Otherwise the
    // block is copied to LDS at two workgroups per CU when table + block fit
    // 80 KiB, else at one per CU when they fit the CU's 160 KiB (re-reading
    // the winners from memory costs more than the lost occupancy: 28.5 ->
    // 18.3 us for 4-bit buckets of a 4096x4096 block row of 8).
    constexpr bool packable = WDT != SKETCH_F32 && (MODE == kEncUniform || MODE == kEncQ4);
    const bool packed = packable && vec && uint64_t(a.R) * uint64_t(a.N) <= kPackedMaxL && tab_bytes <= kStashMax;
    const bool stash2 = vec && !packed && stash_bytes <= kStashMax;
    const bool stash1 = vec && !stash2 && !packed && stash_bytes <= 160 * 1024;
    const bool stash = stash2 || stash1;
    const size_t lds = stash ? stash_bytes : tab_bytes;
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    // Packed words: one workgroup per row block, up to three resident per CU,
    // and the dispatcher hands each freed slot the next block (11008 x 4096 in
    // row blocks of 8, 1376 blocks: 28.1 -> 24.9 us against a persistent grid
    // of two per CU, whose last round is two-thirds full; 28672 x 8192 and
    // 4096 x 4096 unchanged).  The LDS-copy variants stay persistent.
    const int64_t cap = packed ? a.nb : int64_t(ncu) * (stash1 ? 1 : stash ? 2 : 4);
    const unsigned grid = unsigned(a.nb < cap ? a.nb : cap);
    if (stash)
        encode_kernel<WDT, RULE, true, kWinStash, MODE><<<grid, kEncThreads, lds, st>>>(a);
    else if (packed) {
        if constexpr (packable) encode_kernel<WDT, RULE, true, kWinPacked, MODE><<<grid, kEncThreads, lds, st>>>(a);
    } else if (vec)
        encode_kernel<WDT, RULE, true, kWinMemory, MODE><<<grid, kEncThreads, lds, st>>>(a);
    else
        encode_kernel<WDT, RULE, false, kWinMemory, MODE><<<grid, kEncThreads, lds, st>>>(a);
    return launch_status();
}

template <int MODE>
sketch_status launch_rule(const sketch_params* p, const EncArgs& a, bool vec, hipStream_t st) {
    const int rule = p->rule;
    switch (p->w_dtype) {
        case SKETCH_F32:
            return rule == SKETCH_ABSMIN ? launch_typed<SKETCH_F32, SKETCH_ABSMIN, MODE>(a, vec, st)
                                         : launch_typed<SKETCH_F32, SKETCH_ABSMAX, MODE>(a, vec, st);
        case SKETCH_BF16:
            return rule == SKETCH_ABSMIN ? launch_typed<SKETCH_BF16, SKETCH_ABSMIN, MODE>(a, vec, st)
                                         : launch_typed<SKETCH_BF16, SKETCH_ABSMAX, MODE>(a, vec, st);
        case SKETCH_F16:
            return rule == SKETCH_ABSMIN ? launch_typed<SKETCH_F16, SKETCH_ABSMIN, MODE>(a, vec, st)
                                         : launch_typed<SKETCH_F16, SKETCH_ABSMAX, MODE>(a, vec, st);
    }
    return SKETCH_EINVAL;
}

}  // namespace

sketch_status launch_encode(const sketch_params* p, const Shape& s, const void* proj, const void* W,
                            const float* imp, uint16_t* tables, int32_t* status, hipStream_t st) {
    if (s.nb == 0) return SKETCH_OK;
    const ProjLayout L = s.boff ? proj_layout_hash(s.R, s.N)
                         : s.rows > 1 ? proj_layout_rows(s.R, s.N, s.rows) : proj_layout(s.R, s.N, s.Bg);
    EncArgs a;
    a.W = W;
    a.imp = imp;
    a.idx = reinterpret_cast<const uint16_t*>(static_cast<const char*>(proj) + L.idx);
    a.hdr = static_cast<const ProjHeader*>(proj);
    a.S = tables;
    a.status = status;
    a.N = s.N;
    a.nb = s.nb;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.seed = p->seed;
    a.rows = uint32_t(s.rows);
    a.boff = s.boff;
    a.bg_max = uint32_t(s.bg_max);
    a.total = uint64_t(s.nb) * uint64_t(s.Bg);
    a.scales = nullptr;
    a.cpr = uint32_t(s.N / 8);
    a.nchunk = uint32_t(s.R * s.N / 8);
    // Vector path: rows are whole 8-element chunks (16-byte aligned given a
    // 16-byte aligned W), the importance vector is 16-byte aligned, and a
    // block's byte offsets (weights, forward map) fit the 32-bit per-lane
    // offsets it addresses with; larger blocks take the 64-bit scalar path.
    const uint64_t blk_bytes = uint64_t(s.R) * uint64_t(s.N) * (p->w_dtype == SKETCH_F32 ? 4u : 2u);
    const bool vec = (s.N % 8 == 0) && (reinterpret_cast<uintptr_t>(imp) % 16 == 0) &&
                     blk_bytes < (uint64_t(1) << 32);
    if (s.boff) return launch_rule<kEncAlloc>(p, a, vec, st);
    if (s.bits == 4) {
        a.scales = reinterpret_cast<uint16_t*>(reinterpret_cast<char*>(tables) + q4_scales_offset(s));
        return launch_rule<kEncQ4>(p, a, vec, st);
    }
    return s.rows > 1 ? launch_rule<kEncRows>(p, a, vec, st) : launch_rule<kEncUniform>(p, a, vec, st);
}

sketch_status launch_encode_sync(const sketch_params* p, const Shape& s, const void* proj, const void* W,
                                 const float* imp, uint16_t* tables, hipStream_t st) {
    static std::mutex mu;
    static int32_t* word[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SKETCH_EDEVICE;
    if (!word[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_sync_status)) != hipSuccess || !ptr) return SKETCH_EDEVICE;
        word[dev] = static_cast<int32_t*>(ptr);
    }
    clear_status_kernel<<<1, 64, 0, st>>>(word[dev]);
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    const sketch_status rc = launch_encode(p, s, proj, W, imp, tables, word[dev], st);
    if (rc != SKETCH_OK) return rc;
    int32_t flags = 0;
    if (hipMemcpyAsync(&flags, word[dev], sizeof(flags), hipMemcpyDeviceToHost, st) != hipSuccess) return SKETCH_EDEVICE;
    if (hipStreamSynchronize(st) != hipSuccess) return SKETCH_EDEVICE;
    return sketch_encode_status(flags);
}

}  // namespace sketch

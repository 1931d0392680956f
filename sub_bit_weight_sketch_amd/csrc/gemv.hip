// gemv.hip -- decode-batch product Y = X * W_hat^T without materialising W_hat.
//
// "Resumen Técnico" › Metodología §4: W_hat = S * P^T.  Because P is one-hot
// and the same for every row block, the product factorises
//     Y[t][b*R + r] = sum_k S[b][k] * Z[t][r][k],   Z[t][r][k] = sum_{j: k(r*N+j)=k} X[t][j]
// (Resultados › Ablación: the matrix form equals the sequential one).
// Z = P^T x costs R*N adds per token and is independent of M; the product
// with S then reads every bucket table exactly once from HBM.
//
// Kernels
//   gemv_z_kernel      Z (float32) by gathering x through the projection's
//                      inverse map (ascending j: deterministic), plus the
//                      per-256-entry maximum |Z| used for scaling.
//   gemv_mfma_kernel   Y = S * Z^T on matrix cores: A = S rows (binary16,
//                      exact), B = Z * 2^e split into binary16 hi + lo
//                      columns, so every product is exact and accumulation
//                      is float32.  16 row blocks per MFMA tile, K split over
//                      the 4 waves of a workgroup, workgroups persistent over
//                      tiles so Z is staged in LDS once per workgroup.
//   gemv_generic_kernel  float32 VALU fallback for shapes the MFMA kernel
//                      does not take (R not a multiple of 8, Bg not a
//                      multiple of 32, Z too large for LDS, non-finite Z).
#include "common.h"

namespace sketch {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kZThreads = 256;
constexpr int kMfmaThreads = 256;       // 4 waves
constexpr size_t kMfmaLdsBudget = 96 * 1024;

struct GemvWs {
    float* Z;     // [batch][R][Bg]
    float* zmax;  // [batch][nzc]
    int64_t nzc;
};

inline GemvWs gemv_ws(void* ws, const Shape& s, int64_t batch) {
    GemvWs w;
    char* base = static_cast<char*>(ws);
    w.Z = reinterpret_cast<float*>(base);
    w.nzc = (s.R * s.Bg + kZThreads - 1) / kZThreads;
    w.zmax = reinterpret_cast<float*>(base + align256(sizeof(float) * size_t(batch * s.R * s.Bg)));
    return w;
}

__device__ inline bool header_ok(const ProjHeader* h, uint32_t R, uint32_t N, uint32_t Bg) {
    return h->magic == kProjMagic && h->version == kProjVersion && h->R == R && h->N == N && h->Bg == Bg;
}

// ---------------------------------------------------------------------------
// Z = P^T x.  One thread per (t, r, k) segment; a workgroup covers 256
// consecutive segments of one token and records max |Z| over them (+Inf if
// any entry is not finite).  A projection built for another shape poisons Z
// with NaN, which the product propagates to every output.
// ---------------------------------------------------------------------------
template <int XDT>
__global__ __launch_bounds__(kZThreads) void gemv_z_kernel(const void* X, const ProjHeader* hdr,
                                                           const uint32_t* off, const uint16_t* cols,
                                                           float* Z, float* zmax, int64_t N, uint32_t R,
                                                           uint32_t Bg, int64_t nzc) {
    __shared__ float red[kZThreads / 64];
    const int64_t RB = int64_t(R) * Bg;
    const int64_t t = blockIdx.y;
    const int64_t seg = int64_t(blockIdx.x) * kZThreads + threadIdx.x;
    const bool ok = header_ok(hdr, R, uint32_t(N), Bg);
    float z = 0.0f;
    if (seg < RB) {
        if (ok) {
            const uint32_t b = off[seg], e = off[seg + 1];
            for (uint32_t c = b; c < e; ++c) z += load_elem<XDT>(X, t * N + cols[c]);
        } else {
            z = __builtin_nanf("");
        }
        Z[t * RB + seg] = z;
    }
    float m = __builtin_fabsf(z);
    if (!(m <= 3.402823466e38f)) m = __builtin_inff();
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
        for (int w = 1; w < kZThreads / 64; ++w) r = fmaxf(r, red[w]);
        zmax[t * nzc + blockIdx.x] = r;
    }
}

// ---------------------------------------------------------------------------
// Matrix-core product.  Column tile ct (16 MFMA columns) holds token
// t0 + ct / RG and rows rg*8 .. rg*8+7 (rg = ct % RG, RG = R/8): columns
// 0..7 are the hi parts, 8..15 the lo parts of the same rows.
// LDS fragment layout: frag[(s*CT + ct)*64 + lane] = 8 halves, the B operand
// of K-step s (32 buckets) for that lane.
// ---------------------------------------------------------------------------
struct MfmaArgs {
    const uint16_t* S;
    const float* Z;
    const float* zmax;
    float* Y;
    int64_t nb, M, nzc, ntiles;
    uint32_t R, Bg, RG;
    int64_t t0;     // first token of this pass
    int32_t ntok;   // tokens in this pass (<= CT / RG); other columns are zero
};

// float32 dot products of the rows of block b with Z for tokens t0..t0+ntok-1
// (used when Z is not finite or cannot be scaled into binary16 range).
__device__ inline void block_rows_f32(const uint16_t* S, const float* Z, float* Y, int64_t b, int64_t M,
                                      uint32_t R, uint32_t Bg, int64_t t0, int ntok, float* red) {
    const int tid = threadIdx.x;
    const int64_t RB = int64_t(R) * Bg;
    const uint16_t* Sb = S + b * Bg;
    for (int tt = 0; tt < ntok; ++tt) {
        for (uint32_t r = 0; r < R; ++r) {
            const float* z = Z + (t0 + tt) * RB + int64_t(r) * Bg;
            float acc = 0.0f;
            for (uint32_t k = tid; k < Bg; k += blockDim.x) acc += f16_bits_to_f32(Sb[k]) * z[k];
            for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
            if ((tid & 63) == 0) red[tid >> 6] = acc;
            __syncthreads();
            if (tid == 0) {
                float v = 0.0f;
                for (int w = 0; w < int(blockDim.x >> 6); ++w) v += red[w];
                Y[(t0 + tt) * M + b * R + r] = v;
            }
            __syncthreads();
        }
    }
}

template <int CT>
__global__ __launch_bounds__(kMfmaThreads) void gemv_mfma_kernel(MfmaArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char lds_raw[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint32_t nsteps = a.Bg / 32;
    half8* frag = reinterpret_cast<half8*>(lds_raw);
    float4v* red = reinterpret_cast<float4v*>(lds_raw + size_t(nsteps) * CT * 64 * sizeof(half8));
    __shared__ float scale_up[CT], scale_dn[CT];
    __shared__ int finite_ok;

    // Per-token power-of-two scale from max |Z|: max * 2^e lands in [2^14, 2^15).
    if (tid == 0) finite_ok = 1;
    if (tid < CT) {
        scale_up[tid] = 0.0f;   // absent tokens: zero columns
        scale_dn[tid] = 0.0f;
    }
    __syncthreads();
    if (wave == 0) {
        for (int tt = 0; tt < a.ntok; ++tt) {
            const float* zm = a.zmax + (a.t0 + tt) * a.nzc;
            float m = 0.0f;
            for (int64_t c = lane; c < a.nzc; c += 64) m = fmaxf(m, zm[c]);
            for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
            if (lane == 0) {
                int e = 0;
                if (!(m <= 3.402823466e38f)) {
                    finite_ok = 0;
                } else if (m > 0.0f) {
                    e = 14 - ilogbf(m);
                    if (e > 120 || e < -120) finite_ok = 0;
                }
                for (int g = 0; g < int(a.RG); ++g) {
                    scale_up[tt * a.RG + g] = ldexpf(1.0f, e);
                    scale_dn[tt * a.RG + g] = ldexpf(1.0f, -e);
                }
            }
        }
    }
    __syncthreads();
    if (!finite_ok) {
        float* red32 = reinterpret_cast<float*>(lds_raw);
        for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x)
            for (int64_t b = tile * 16; b < tile * 16 + 16 && b < a.nb; ++b)
                block_rows_f32(a.S, a.Z, a.Y, b, a.M, a.R, a.Bg, a.t0, a.ntok, red32);
        return;
    }

    // Stage B fragments.
    const int64_t RB = int64_t(a.R) * a.Bg;
    const uint32_t nfrag = nsteps * CT * 64;
    for (uint32_t f = tid; f < nfrag; f += kMfmaThreads) {
        const uint32_t l = f & 63, ct = (f >> 6) % CT, s = (f >> 6) / CT;
        const uint32_t col = l & 15;
        const uint32_t tt = ct / a.RG, rg = ct % a.RG;
        const uint32_t r = rg * 8 + (col & 7);
        const uint32_t k0 = s * 32 + (l >> 4) * 8;
        float4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
        if (int(tt) < a.ntok) {
            const float* zp = a.Z + (a.t0 + tt) * RB + int64_t(r) * a.Bg + k0;
            z0 = *reinterpret_cast<const float4*>(zp);
            z1 = *reinterpret_cast<const float4*>(zp + 4);
        }
        const float zs[8] = {z0.x, z0.y, z0.z, z0.w, z1.x, z1.y, z1.z, z1.w};
        const float sc = scale_up[ct];
        half8 h;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = zs[i] * sc;
            const _Float16 hi = static_cast<_Float16>(v);
            h[i] = (col < 8) ? hi : static_cast<_Float16>(v - static_cast<float>(hi));
        }
        frag[f] = h;
    }
    __syncthreads();

    for (int64_t tile = blockIdx.x; tile < a.ntiles; tile += gridDim.x) {
        const int64_t b0 = tile * 16;
        const int64_t row = b0 + (lane & 15);
        const bool row_ok = row < a.nb;
        const uint16_t* srow = a.S + row * int64_t(a.Bg) + (lane >> 4) * 8;
        float4v acc[CT];
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[c] = float4v{0.f, 0.f, 0.f, 0.f};

        uint32_t s = wave;
        for (; s + 12 < nsteps; s += 16) {
            half8 av[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                av[u] = row_ok ? __builtin_nontemporal_load(reinterpret_cast<const half8*>(srow + (s + 4 * u) * 32))
                               : half8{};
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int c = 0; c < CT; ++c)
                    acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av[u], frag[((s + 4 * u) * CT + c) * 64 + lane],
                                                                    acc[c], 0, 0, 0);
        }
        for (; s < nsteps; s += 4) {
            half8 av = row_ok ? __builtin_nontemporal_load(reinterpret_cast<const half8*>(srow + s * 32)) : half8{};
#pragma unroll
            for (int c = 0; c < CT; ++c)
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(av, frag[(s * CT + c) * 64 + lane], acc[c], 0, 0, 0);
        }
#pragma unroll
        for (int c = 0; c < CT; ++c) red[(wave * CT + c) * 64 + lane] = acc[c];
        __syncthreads();
        // Sum the 4 K-slices; combine hi + lo columns; unscale; store.
        for (int c = wave; c < CT; c += 4) {
            float4v v = red[(0 * CT + c) * 64 + lane];
#pragma unroll
            for (int w = 1; w < 4; ++w) v += red[(w * CT + c) * 64 + lane];
            float4v p;
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = __shfl_xor(v[i], 8);
            const uint32_t col = lane & 15;
            if (col < 8 && int(c / a.RG) < a.ntok) {
                const uint32_t tt = c / a.RG, rg = c % a.RG;
                const uint32_t r = rg * 8 + col;
                float* yrow = a.Y + (a.t0 + tt) * a.M;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t blk = b0 + (lane >> 4) * 4 + i;
                    if (blk < a.nb) yrow[blk * a.R + r] = (v[i] + p[i]) * scale_dn[c];
                }
            }
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Generic float32 fallback: one workgroup per block, one token at a time.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gemv_generic_kernel(const uint16_t* S, const float* Z, float* Y,
                                                           int64_t nb, int64_t M, uint32_t R, uint32_t Bg,
                                                           int64_t batch) {
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
                if (tid == 0) Y[t * M + b * R + r] = red[0] + red[1] + red[2] + red[3];
                __syncthreads();
            }
        }
    }
}

template <int CT>
void launch_mfma(const MfmaArgs& a, size_t lds, int grid, hipStream_t st) {
    gemv_mfma_kernel<CT><<<grid, kMfmaThreads, lds, st>>>(a);
}

int num_cus() {
    int dev = 0, ncu = 256;
    if (hipGetDevice(&dev) == hipSuccess)
        (void)hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    return ncu;
}

}  // namespace

size_t gemv_workspace_bytes(const Shape& s, int64_t batch) {
    const int64_t nzc = (s.R * s.Bg + kZThreads - 1) / kZThreads;
    return align256(sizeof(float) * size_t(batch * s.R * s.Bg)) + align256(sizeof(float) * size_t(batch * nzc));
}

sketch_status launch_gemv(const sketch_params* p, const Shape& s, const void* proj, const uint16_t* tables,
                          const void* X, sketch_dtype xdt, int64_t batch, float* Y, void* ws, hipStream_t st) {
    (void)p;
    const ProjLayout L = proj_layout(s.R, s.N, s.Bg);
    const char* pb = static_cast<const char*>(proj);
    const auto* hdr = reinterpret_cast<const ProjHeader*>(pb);
    const auto* off = reinterpret_cast<const uint32_t*>(pb + L.off);
    const auto* cols = reinterpret_cast<const uint16_t*>(pb + L.cols);
    GemvWs w = gemv_ws(ws, s, batch);

    dim3 zg(unsigned(w.nzc), unsigned(batch));
    switch (xdt) {
        case SKETCH_F32:
            gemv_z_kernel<SKETCH_F32><<<zg, kZThreads, 0, st>>>(X, hdr, off, cols, w.Z, w.zmax, s.N, uint32_t(s.R),
                                                                 uint32_t(s.Bg), w.nzc);
            break;
        case SKETCH_BF16:
            gemv_z_kernel<SKETCH_BF16><<<zg, kZThreads, 0, st>>>(X, hdr, off, cols, w.Z, w.zmax, s.N,
                                                                  uint32_t(s.R), uint32_t(s.Bg), w.nzc);
            break;
        case SKETCH_F16:
            gemv_z_kernel<SKETCH_F16><<<zg, kZThreads, 0, st>>>(X, hdr, off, cols, w.Z, w.zmax, s.N, uint32_t(s.R),
                                                                 uint32_t(s.Bg), w.nzc);
            break;
    }
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;

    // Matrix-core path: R a multiple of 8 (at most 16 row groups), Bg a
    // multiple of 32, and the fragments of RG column tiles fit the LDS budget.
    const int64_t RG = s.R / 8;
    auto lds_for = [&](int ct) { return size_t(s.Bg) * ct * 32 + size_t(4 * ct * 64 * 16); };
    int CT = 0;
    if (s.R % 8 == 0 && RG <= 16 && s.Bg % 32 == 0) {
        for (int ct : {16, 8, 4, 2, 1}) {
            if (ct < RG || ct % RG != 0 || lds_for(ct) > kMfmaLdsBudget) continue;
            CT = ct;
            // no wider than the batch needs
            while (CT > RG && (CT / 2) >= RG * batch) CT /= 2;
            break;
        }
    }
    if (CT == 0) {
        int grid = int(s.nb < 4096 ? s.nb : 4096);
        gemv_generic_kernel<<<grid, 256, 0, st>>>(tables, w.Z, Y, s.nb, s.M, uint32_t(s.R), uint32_t(s.Bg), batch);
        return launch_status();
    }

    const int64_t TB = CT / RG;
    MfmaArgs a;
    a.S = tables;
    a.Z = w.Z;
    a.zmax = w.zmax;
    a.Y = Y;
    a.nb = s.nb;
    a.M = s.M;
    a.nzc = w.nzc;
    a.ntiles = (s.nb + 15) / 16;
    a.R = uint32_t(s.R);
    a.Bg = uint32_t(s.Bg);
    a.RG = uint32_t(RG);
    const int grid = int(a.ntiles < int64_t(num_cus()) ? a.ntiles : int64_t(num_cus()));
    const size_t lds = lds_for(CT);
    for (int64_t t0 = 0; t0 < batch; t0 += TB) {
        a.t0 = t0;
        a.ntok = int32_t(batch - t0 < TB ? batch - t0 : TB);
        switch (CT) {
            case 1: launch_mfma<1>(a, lds, grid, st); break;
            case 2: launch_mfma<2>(a, lds, grid, st); break;
            case 4: launch_mfma<4>(a, lds, grid, st); break;
            case 8: launch_mfma<8>(a, lds, grid, st); break;
            default: launch_mfma<16>(a, lds, grid, st); break;
        }
        if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    }
    return SKETCH_OK;
}

}  // namespace sketch

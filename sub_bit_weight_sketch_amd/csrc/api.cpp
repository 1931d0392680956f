// api.cpp -- the C ABI declared in include/sketch.h: validation and dispatch.
//
// Budget (Resumen Técnico › Resultados: 0.5 bits per weight): one binary16
// bucket per 16/bpw weights, Bg = R*N*bpw/16 buckets per row block.
#include <cmath>
#include <cstdint>
#include <algorithm>
#include <vector>

#include "common.h"

using namespace sketch;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

sketch_status sketch::validate_params(const sketch_params* p, Shape* s) {
    if (!p) return SKETCH_EINVAL;
    if (p->M < 0 || p->N < 1 || p->N > SKETCH_MAX_N || p->R < 1) return SKETCH_EINVAL;
    if (p->M % p->R != 0) return SKETCH_EINVAL;
    if (!(p->bpw > 0.0) || !std::isfinite(p->bpw)) return SKETCH_EINVAL;
    if (p->rule != SKETCH_ABSMIN && p->rule != SKETCH_ABSMAX) return SKETCH_EINVAL;
    if (p->w_dtype != SKETCH_F32 && p->w_dtype != SKETCH_BF16 && p->w_dtype != SKETCH_F16) return SKETCH_EINVAL;
    const double rn = double(p->R) * double(p->N);
    // kernels address a block's weights and its forward map (2 bytes per
    // weight) with 32-bit byte offsets from the block's base
    const double wes = p->w_dtype == SKETCH_F32 ? 4.0 : 2.0;
    if (rn * wes >= 4294967296.0) return SKETCH_EINVAL;
    const int32_t bits = p->bucket_bits == 0 ? 16 : p->bucket_bits;
    if (bits != 16 && bits != 4) return SKETCH_EINVAL;
    const double bg = rn * p->bpw / double(bits);
    if (bits == 16 && (bg != std::floor(bg) || bg < 1.0 || bg > double(SKETCH_MAX_BG))) return SKETCH_EINVAL;
    if (bits == 4 && (bg != std::floor(bg) || bg < 2.0 || bg > double(SKETCH_MAX_BG4) || std::fmod(bg, 2.0) != 0.0))
        return SKETCH_EINVAL;
    const int64_t rows = p->rows <= 1 ? 1 : p->rows;
    if (p->rows < 0 || rows > SKETCH_MAX_ROWS || int64_t(bg) % rows != 0) return SKETCH_EINVAL;
    s->M = p->M;
    s->N = p->N;
    s->R = p->R;
    s->Bg = int64_t(bg);
    s->nb = p->M / p->R;
    s->rows = rows;
    s->boff = p->block_offsets;
    s->bg_max = 0;
    s->bits = bits;
    if (bits == 4 && (rows != 1 || p->block_offsets)) return SKETCH_EINVAL;
    if (p->block_offsets) {   // importance-aware allocation
        if (rows != 1 || p->block_bg_max < 1 || p->block_bg_max > SKETCH_MAX_BG) return SKETCH_EINVAL;
        if (reinterpret_cast<uintptr_t>(p->block_offsets) & 3u) return SKETCH_EINVAL;
        if (double(s->nb) * bg >= 4294967296.0) return SKETCH_EINVAL;
        s->bg_max = p->block_bg_max;
    }
    return SKETCH_OK;
}

namespace {

sketch_status validate(const sketch_params* p, Shape* s) { return validate_params(p, s); }

bool valid_dtype(sketch_dtype d) { return d == SKETCH_F32 || d == SKETCH_BF16 || d == SKETCH_F16; }

// optional: whether to count the workspace that only speeds the call up
sketch_status workspace_bytes(const sketch_params* p, int64_t batch, sketch_dtype x_dtype, bool optional,
                              size_t* bytes) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!bytes || batch < 0 || !valid_dtype(x_dtype)) return SKETCH_EINVAL;
    if (batch == 0 || s.nb == 0)
        *bytes = 0;
    else if (s.rows > 1)   // the multi-row prefill's K split
        *bytes = optional ? rows_gemm_split_bytes(p, s, x_dtype, batch) : 0;
    else if (s.boff || s.bits == 4 || gemm_supported(p, s, x_dtype, batch))
        *bytes = 0;
    else
        *bytes = gemv_workspace_bytes(s, batch, x_dtype);
    return SKETCH_OK;
}
}  // namespace

sketch_status sketch::required_workspace_bytes(const sketch_params* p, int64_t batch, sketch_dtype x_dtype,
                                               size_t* bytes) {
    return workspace_bytes(p, batch, x_dtype, false, bytes);
}

extern "C" {

sketch_status sketch_layout(const sketch_params* p, int64_t* num_blocks, int64_t* Bg, size_t* table_bytes) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (num_blocks) *num_blocks = s.nb;
    if (Bg) *Bg = s.Bg;
    if (table_bytes)
        *table_bytes = s.bits == 4 ? q4_scales_offset(s) + size_t(s.nb) * 2 : size_t(s.nb) * size_t(s.Bg) * 2;
    return SKETCH_OK;
}

sketch_status sketch_projection_bytes(const sketch_params* p, size_t* bytes) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!bytes) return SKETCH_EINVAL;
    *bytes = s.boff       ? proj_layout_hash(s.R, s.N).total
             : s.rows > 1 ? proj_layout_rows(s.R, s.N, s.rows).total
                          : proj_layout(s.R, s.N, s.Bg).total;
    return SKETCH_OK;
}

sketch_status sketch_projection_build(const sketch_params* p, void* proj, size_t proj_bytes, void* stream) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!proj || !aligned16(proj)) return SKETCH_EINVAL;
    if (s.boff) {
        if (proj_bytes < proj_layout_hash(s.R, s.N).total) return SKETCH_ESMALL;
        return launch_projection_build_hash(p, s, proj, static_cast<hipStream_t>(stream));
    }
    if (s.rows > 1) {
        if (proj_bytes < proj_layout_rows(s.R, s.N, s.rows).total) return SKETCH_ESMALL;
        return launch_projection_build_rows(p, s, proj, static_cast<hipStream_t>(stream));
    }
    if (proj_bytes < proj_layout(s.R, s.N, s.Bg).total) return SKETCH_ESMALL;
    return launch_projection_build(p, s, proj, static_cast<hipStream_t>(stream));
}

sketch_status sketch_encode(const sketch_params* p, const void* proj, const void* W, const float* importance,
                            uint16_t* tables, int32_t* status_dev, void* stream) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!proj || !aligned16(proj) || (reinterpret_cast<uintptr_t>(status_dev) & 3u)) return SKETCH_EINVAL;
    if (importance && (reinterpret_cast<uintptr_t>(importance) & 3u)) return SKETCH_EINVAL;
    if (s.nb == 0) return SKETCH_OK;
    if (!W || !tables || !aligned16(W) || !aligned16(tables)) return SKETCH_EINVAL;
    if (!status_dev) return launch_encode_sync(p, s, proj, W, importance, tables, static_cast<hipStream_t>(stream));
    return launch_encode(p, s, proj, W, importance, tables, status_dev, static_cast<hipStream_t>(stream));
}

sketch_status sketch_encode_status(int32_t flags) {
    if (flags & (SKETCH_FLAG_IMPORTANCE | SKETCH_FLAG_PROJECTION | SKETCH_FLAG_ALLOCATION)) return SKETCH_EINVAL;
    if (flags & SKETCH_FLAG_WEIGHT_RANGE) return SKETCH_ERANGE;
    if (flags) return SKETCH_EINVAL;
    return SKETCH_OK;
}

sketch_status sketch_workspace_bytes(const sketch_params* p, int64_t batch, sketch_dtype x_dtype, size_t* bytes) {
    return workspace_bytes(p, batch, x_dtype, true, bytes);
}

sketch_status sketch_matmul(const sketch_params* p, const void* proj, const uint16_t* tables, const void* X,
                            sketch_dtype x_dtype, int64_t batch, float* Y, void* workspace, size_t workspace_bytes,
                            void* stream) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (batch < 0 || !valid_dtype(x_dtype)) return SKETCH_EINVAL;
    if (batch == 0 || s.nb == 0) return SKETCH_OK;
    if (!proj || !tables || !X || !Y || !aligned16(proj) || !aligned16(tables) || !aligned16(X) || !aligned16(Y))
        return SKETCH_EINVAL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (s.boff) return launch_matmul_alloc(p, s, proj, tables, X, x_dtype, batch, Y, st);
    if (s.bits == 4) return launch_matmul_q4(p, s, proj, tables, X, x_dtype, batch, Y, st);
    if (s.rows > 1) return launch_matmul_rows(p, s, proj, tables, X, x_dtype, batch, Y, workspace, workspace_bytes, st);
    if (gemm_supported(p, s, x_dtype, batch)) return launch_gemm(p, s, proj, tables, X, batch, Y, st);
    const size_t need = gemv_workspace_bytes(s, batch, x_dtype);
    if (need > 0) {
        if (!workspace || !aligned16(workspace)) return SKETCH_EINVAL;
        if (workspace_bytes < need) return SKETCH_ESMALL;
    }
    return launch_gemv(p, s, proj, tables, X, x_dtype, batch, Y, workspace, st);
}

sketch_status sketch_decode(const sketch_params* p, const void* proj, const uint16_t* tables, void* out,
                            sketch_dtype out_dtype, void* stream) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!valid_dtype(out_dtype)) return SKETCH_EINVAL;
    if (s.nb == 0) return SKETCH_OK;
    if (!proj || !tables || !out || !aligned16(proj) || !aligned16(tables) || !aligned16(out)) return SKETCH_EINVAL;
    if (s.boff) return launch_decode_alloc(p, s, proj, tables, out, out_dtype, false, static_cast<hipStream_t>(stream));
    if (s.bits == 4) return launch_decode_q4(p, s, proj, tables, out, out_dtype, false, static_cast<hipStream_t>(stream));
    return launch_decode(p, s, proj, tables, out, out_dtype, static_cast<hipStream_t>(stream));
}

sketch_status sketch_decode_hashed(const sketch_params* p, const uint16_t* tables, void* out, sketch_dtype out_dtype,
                                   void* stream) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!valid_dtype(out_dtype)) return SKETCH_EINVAL;
    if (s.nb == 0) return SKETCH_OK;
    if (!tables || !out || !aligned16(tables) || !aligned16(out)) return SKETCH_EINVAL;
    if (s.boff)
        return launch_decode_alloc(p, s, nullptr, tables, out, out_dtype, true, static_cast<hipStream_t>(stream));
    if (s.bits == 4)
        return launch_decode_q4(p, s, nullptr, tables, out, out_dtype, true, static_cast<hipStream_t>(stream));
    return launch_decode_hashed(p, s, tables, out, out_dtype, static_cast<hipStream_t>(stream));
}

sketch_status sketch_block_importance(const sketch_params* p, const void* W, const float* a2, float* scores,
                                      void* stream) {
    if (!p) return SKETCH_EINVAL;
    if (p->M < 0 || p->N < 1 || p->N > SKETCH_MAX_N || p->R < 1 || p->M % p->R != 0) return SKETCH_EINVAL;
    if (p->w_dtype != SKETCH_F32 && p->w_dtype != SKETCH_BF16 && p->w_dtype != SKETCH_F16) return SKETCH_EINVAL;
    if (double(p->R) * double(p->N) >= 4294967296.0) return SKETCH_EINVAL;
    Shape s{};
    s.M = p->M;
    s.N = p->N;
    s.R = p->R;
    s.nb = p->M / p->R;
    if (s.nb == 0) return SKETCH_OK;
    if (!W || !a2 || !scores || !aligned16(W) || (reinterpret_cast<uintptr_t>(a2) & 3u) ||
        (reinterpret_cast<uintptr_t>(scores) & 3u))
        return SKETCH_EINVAL;
    return launch_block_importance(p, s, W, a2, scores, static_cast<hipStream_t>(stream));
}

sketch_status sketch_alloc_plan(int64_t nb, int64_t total, int64_t lo, const double* scores, uint32_t* offsets,
                                int32_t* bg_max) {
    if (nb < 1 || lo < 1 || !scores || !offsets || total < nb * lo || total >= 4294967296LL) return SKETCH_EINVAL;
    double sum = 0.0;
    for (int64_t b = 0; b < nb; ++b) {
        if (!std::isfinite(scores[b]) || scores[b] < 0.0) return SKETCH_EINVAL;
        sum += scores[b];
    }
    if (!std::isfinite(sum)) return SKETCH_EINVAL;
    const int64_t E = total - nb * lo;
    std::vector<int64_t> cnt(size_t(nb), 0);
    std::vector<double> rem(size_t(nb), 0.0);
    std::vector<int64_t> order(static_cast<size_t>(nb));
    int64_t left = E;
    for (int64_t b = 0; b < nb; ++b) {
        const double q = sum > 0.0 ? (double(E) * scores[b]) / sum : double(E) / double(nb);
        const double f = std::floor(q);
        cnt[size_t(b)] = int64_t(f);
        rem[size_t(b)] = q - f;
        left -= cnt[size_t(b)];
        order[size_t(b)] = b;
    }
    // leftover units to the largest remainders (ties: lower block); a
    // rounding overshoot is taken back from the smallest (ties: higher block)
    if (left != 0) {
        std::vector<int64_t> idx(order);
        auto by_rem_desc = [&](int64_t a, int64_t c) {
            return rem[size_t(a)] > rem[size_t(c)] || (rem[size_t(a)] == rem[size_t(c)] && a < c);
        };
        std::sort(idx.begin(), idx.end(), by_rem_desc);
        if (left > 0) {
            for (int64_t u = 0; u < left; ++u) cnt[size_t(idx[size_t(u)])] += 1;
        } else {
            int64_t give = -left;
            for (int64_t u = nb - 1; u >= 0 && give > 0; --u)
                if (cnt[size_t(idx[size_t(u)])] > 0) {
                    cnt[size_t(idx[size_t(u)])] -= 1;
                    --give;
                }
            if (give > 0) return SKETCH_EINVAL;
        }
    }
    int64_t mx = 0, at = 0;
    offsets[0] = 0;
    for (int64_t b = 0; b < nb; ++b) {
        const int64_t c = lo + cnt[size_t(b)];
        if (c > SKETCH_MAX_BG) return SKETCH_EINVAL;
        mx = c > mx ? c : mx;
        at += c;
        offsets[b + 1] = uint32_t(at);
    }
    if (bg_max) *bg_max = int32_t(mx);
    return SKETCH_OK;
}

const char* sketch_status_str(sketch_status s) {
    switch (s) {
        case SKETCH_OK: return "ok";
        case SKETCH_EINVAL: return "invalid argument";
        case SKETCH_ERANGE: return "weight out of binary16 range";
        case SKETCH_EDEVICE: return "device error";
        case SKETCH_ESMALL: return "buffer too small";
        case SKETCH_ENOSPACE: return "product needs more than the static scratch";
    }
    return "unknown status";
}

}  // extern "C"

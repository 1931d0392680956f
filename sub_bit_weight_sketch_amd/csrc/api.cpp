// api.cpp -- the C ABI declared in include/sketch.h: validation and dispatch.
//
// Budget (Resumen Técnico › Resultados: 0.5 bits per weight): one binary16
// bucket per 16/bpw weights, Bg = R*N*bpw/16 buckets per row block.
#include <cmath>
#include <cstdint>

#include "common.h"

using namespace sketch;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

sketch_status validate(const sketch_params* p, Shape* s) {
    if (!p) return SKETCH_EINVAL;
    if (p->M < 0 || p->N < 1 || p->N > SKETCH_MAX_N || p->R < 1) return SKETCH_EINVAL;
    if (p->M % p->R != 0) return SKETCH_EINVAL;
    if (!(p->bpw > 0.0) || !std::isfinite(p->bpw)) return SKETCH_EINVAL;
    if (p->rule != SKETCH_ABSMIN && p->rule != SKETCH_ABSMAX) return SKETCH_EINVAL;
    if (p->w_dtype != SKETCH_F32 && p->w_dtype != SKETCH_BF16 && p->w_dtype != SKETCH_F16) return SKETCH_EINVAL;
    const double rn = double(p->R) * double(p->N);
    if (rn >= 4294967296.0) return SKETCH_EINVAL;
    const double bg = rn * p->bpw / 16.0;
    if (bg != std::floor(bg) || bg < 1.0 || bg > double(SKETCH_MAX_BG)) return SKETCH_EINVAL;
    const int64_t rows = p->rows <= 1 ? 1 : p->rows;
    if (p->rows < 0 || rows > SKETCH_MAX_ROWS || int64_t(bg) % rows != 0) return SKETCH_EINVAL;
    s->M = p->M;
    s->N = p->N;
    s->R = p->R;
    s->Bg = int64_t(bg);
    s->nb = p->M / p->R;
    s->rows = rows;
    return SKETCH_OK;
}

bool valid_dtype(sketch_dtype d) { return d == SKETCH_F32 || d == SKETCH_BF16 || d == SKETCH_F16; }

}  // namespace

extern "C" {

sketch_status sketch_layout(const sketch_params* p, int64_t* num_blocks, int64_t* Bg, size_t* table_bytes) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (num_blocks) *num_blocks = s.nb;
    if (Bg) *Bg = s.Bg;
    if (table_bytes) *table_bytes = size_t(s.nb) * size_t(s.Bg) * 2;
    return SKETCH_OK;
}

sketch_status sketch_projection_bytes(const sketch_params* p, size_t* bytes) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!bytes) return SKETCH_EINVAL;
    *bytes = s.rows > 1 ? proj_layout_rows(s.R, s.N, s.rows).total : proj_layout(s.R, s.N, s.Bg).total;
    return SKETCH_OK;
}

sketch_status sketch_projection_build(const sketch_params* p, void* proj, size_t proj_bytes, void* stream) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!proj || !aligned16(proj)) return SKETCH_EINVAL;
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
    if (!proj || !status_dev || !aligned16(proj) || (reinterpret_cast<uintptr_t>(status_dev) & 3u)) return SKETCH_EINVAL;
    if (importance && (reinterpret_cast<uintptr_t>(importance) & 3u)) return SKETCH_EINVAL;
    if (s.nb == 0) return SKETCH_OK;
    if (!W || !tables || !aligned16(W) || !aligned16(tables)) return SKETCH_EINVAL;
    return launch_encode(p, s, proj, W, importance, tables, status_dev, static_cast<hipStream_t>(stream));
}

sketch_status sketch_encode_status(int32_t flags) {
    if (flags & (SKETCH_FLAG_IMPORTANCE | SKETCH_FLAG_PROJECTION)) return SKETCH_EINVAL;
    if (flags & SKETCH_FLAG_WEIGHT_RANGE) return SKETCH_ERANGE;
    if (flags) return SKETCH_EINVAL;
    return SKETCH_OK;
}

sketch_status sketch_workspace_bytes(const sketch_params* p, int64_t batch, sketch_dtype x_dtype, size_t* bytes) {
    Shape s;
    sketch_status rc = validate(p, &s);
    if (rc != SKETCH_OK) return rc;
    if (!bytes || batch < 0 || !valid_dtype(x_dtype)) return SKETCH_EINVAL;
    if (batch == 0 || s.nb == 0 || s.rows > 1 || gemm_supported(p, s, x_dtype, batch))
        *bytes = 0;
    else
        *bytes = gemv_workspace_bytes(s, batch, x_dtype);
    return SKETCH_OK;
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
    if (s.rows > 1) return launch_matmul_rows(p, s, proj, tables, X, x_dtype, batch, Y, st);
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
    return launch_decode_hashed(p, s, tables, out, out_dtype, static_cast<hipStream_t>(stream));
}

const char* sketch_status_str(sketch_status s) {
    switch (s) {
        case SKETCH_OK: return "ok";
        case SKETCH_EINVAL: return "invalid argument";
        case SKETCH_ERANGE: return "weight out of binary16 range";
        case SKETCH_EDEVICE: return "device error";
        case SKETCH_ESMALL: return "buffer too small";
    }
    return "unknown status";
}

}  // extern "C"

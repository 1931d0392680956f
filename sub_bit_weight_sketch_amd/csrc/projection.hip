// projection.hip -- build the index form of the one-hot projection P.
//
// "Resumen Técnico" › Metodología §4: compression and decompression go
// through a projection matrix P whose storage is negligible with a two-level
// cache.  P is one-hot: row l (a local index l = r*N + j inside a row block)
// has its single 1 in column k(l).  The map does not depend on the block, so
// this buffer is the first cache level: built once per (R, N, Bg, seed) and
// shared by every block of every linear of that shape.
//
// Six small launches (a one-time cost per shape):
//   1. clear the per-segment counters and the header (an invalid magic);
//   2. forward map idx[l] = k(l) and segment sizes (r, k(l)) by integer atomics;
//   3. exclusive scan of the sizes -> CSR offsets (one workgroup);
//   4. scatter every j into its segment (atomic cursor: arbitrary order);
//   5. sort every segment ascending, which makes the result deterministic;
//   6. write the header.
// The header is valid only once everything before it on the stream has
// run, so a kernel that checks it never accepts a half-built buffer.
#include "common.h"

namespace sketch {
namespace {

__global__ void proj_clear_kernel(uint32_t* cnt, int64_t n, ProjHeader* hdr) {
    int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < n) cnt[i] = 0;
    if (i == 0) *hdr = ProjHeader{0, 0, 0, 0, 0, 0, {0, 0}};
}

__global__ void proj_header_kernel(ProjHeader* hdr, ProjHeader h) {
    if (threadIdx.x == 0) *hdr = h;
}

__global__ void proj_index_kernel(uint16_t* idx, uint32_t* cnt, int64_t R, int64_t N, uint32_t Bg,
                                  uint32_t seed) {
    int64_t l = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (l >= R * N) return;
    uint32_t k = bucket_of(uint32_t(l), seed, Bg);
    idx[l] = uint16_t(k);
    int64_t r = l / N;
    atomicAdd(&cnt[r * Bg + k], 1u);
}

// Exclusive scan of n counters into off[0..n]; one workgroup of 1024 threads,
// each owning a contiguous run.  Also resets the counters (reused as cursors).
__global__ __launch_bounds__(1024) void proj_scan_kernel(uint32_t* cnt, uint32_t* off, int64_t n) {
    __shared__ uint32_t part[1024];
    const int t = threadIdx.x;
    const int64_t per = (n + 1023) / 1024;
    const int64_t b = t * per, e = (b + per < n) ? b + per : n;
    uint32_t s = 0;
    for (int64_t i = b; i < e; ++i) s += cnt[i];
    part[t] = s;
    __syncthreads();
    // Hillis-Steele inclusive scan over the 1024 partial sums.
    for (int d = 1; d < 1024; d <<= 1) {
        uint32_t v = (t >= d) ? part[t - d] : 0;
        __syncthreads();
        part[t] += v;
        __syncthreads();
    }
    uint32_t run = part[t] - s;  // exclusive prefix of this run
    for (int64_t i = b; i < e; ++i) {
        uint32_t c = cnt[i];
        off[i] = run;
        run += c;
        cnt[i] = 0;
    }
    if (t == 1023) off[n] = part[1023];
}

__global__ void proj_fill_kernel(const uint16_t* idx, const uint32_t* off, uint32_t* cur, uint16_t* cols,
                                 int64_t R, int64_t N, uint32_t Bg) {
    int64_t l = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (l >= R * N) return;
    int64_t r = l / N, j = l - r * N;
    int64_t seg = r * Bg + idx[l];
    uint32_t pos = off[seg] + atomicAdd(&cur[seg], 1u);
    cols[pos] = uint16_t(j);
}

__global__ void proj_sort_kernel(const uint32_t* off, uint16_t* cols, int64_t nseg) {
    int64_t s = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (s >= nseg) return;
    const uint32_t b = off[s], e = off[s + 1];
    for (uint32_t i = b + 1; i < e; ++i) {  // insertion sort; segments hold ~N/Bg entries
        uint16_t v = cols[i];
        uint32_t p = i;
        while (p > b && cols[p - 1] > v) {
            cols[p] = cols[p - 1];
            --p;
        }
        cols[p] = v;
    }
}

inline unsigned grid_for(int64_t n, int threads) { return unsigned((n + threads - 1) / threads); }

}  // namespace

sketch_status launch_proj_header(void* proj, const ProjHeader& h, hipStream_t st) {
    proj_header_kernel<<<1, 64, 0, st>>>(static_cast<ProjHeader*>(proj), h);
    return launch_status();
}

sketch_status launch_projection_build(const sketch_params* p, const Shape& s, void* proj, hipStream_t st) {
    const ProjLayout L = proj_layout(s.R, s.N, s.Bg);
    char* base = static_cast<char*>(proj);
    auto* hdr = reinterpret_cast<ProjHeader*>(base);
    auto* idx = reinterpret_cast<uint16_t*>(base + L.idx);
    auto* off = reinterpret_cast<uint32_t*>(base + L.off);
    auto* cols = reinterpret_cast<uint16_t*>(base + L.cols);
    auto* cnt = reinterpret_cast<uint32_t*>(base + L.cnt);
    const int64_t nseg = s.R * s.Bg, npos = s.R * s.N;
    ProjHeader h{kProjMagic, kProjVersion, uint32_t(s.R), uint32_t(s.N), uint32_t(s.Bg), p->seed, {0, 0}};

    proj_clear_kernel<<<grid_for(nseg > 1 ? nseg : 1, 256), 256, 0, st>>>(cnt, nseg, hdr);
    proj_index_kernel<<<grid_for(npos, 256), 256, 0, st>>>(idx, cnt, s.R, s.N, uint32_t(s.Bg), p->seed);
    proj_scan_kernel<<<1, 1024, 0, st>>>(cnt, off, nseg);
    proj_fill_kernel<<<grid_for(npos, 256), 256, 0, st>>>(idx, off, cnt, cols, s.R, s.N, uint32_t(s.Bg));
    proj_sort_kernel<<<grid_for(nseg, 256), 256, 0, st>>>(off, cols, nseg);
    if (launch_status() != SKETCH_OK) return SKETCH_EDEVICE;
    return launch_proj_header(proj, h, st);
}

}  // namespace sketch

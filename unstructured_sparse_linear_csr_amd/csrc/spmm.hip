// CSR SpMM for gfx950: C = A * B with A sparse (CSR) and B, C dense row-major
// ("Sparse GPU Kernels for Deep Learning", summary card, "Summary": SpMM on
// plain CSR using 1-D tiling, vector memory access on misaligned sparse data,
// and load balancing decoupled from the parallelisation).
//
// Mapping.  One wavefront (= one workgroup) owns a 1-D output strip: kRpw
// consecutive work slots (rows in row_indices order) by one column tile of
// kLpr * kVec columns.  Each slot is served by a group of kLpr lanes; a lane
// owns kVec adjacent output columns and keeps their sums in registers, so C is
// written exactly once, with no atomics and no split over k.
//
// Staging.  A group copies its row's (column, value) pairs into LDS one window
// of 4 * kLpr entries at a time.  On the vector path each lane reads 4 entries
// with one dwordx4 load of col_indices and one of values, starting from the
// row's first entry rounded down to a multiple of 4; entries before the row's
// start (the misaligned prefix) and after its end are staged but skipped.  The
// first window thus costs at most one extra 16-byte segment per row, and every
// CSR load is a full aligned vector.
//
// Hot loop.  Per staged entry each lane issues one dwordx4 load of its kVec
// columns of the B row the entry selects, then kVec FMAs.  kUnroll entries are
// loaded before any is used so that many gathers are in flight per wave.  The
// staged B-row offset is kept in bytes as a 32-bit value when k*n < 2^30, so
// the gather is a scalar-base plus 32-bit vector-offset load.
//
// Order of summation: entries of a row in CSR order, sequentially, with fused
// multiply-add -- deterministic, and identical whatever row order is used.
#include "sp_device.h"
#include "sp_launch.h"

namespace spk {

namespace {

constexpr int kSpmmUnroll = 8;

struct SpmmParams {
    int m, n, nnz, row_blocks;
    const int *row_indices;
    const int *row_offsets;
    const int *col_indices;
    const float *values;
    const float *b;
    float *c;
    long long stride_values, stride_b, stride_c;
};

template <int kVec> struct Vec;
template <> struct Vec<4> {
    using T = float4;
    static __device__ __forceinline__ T zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
    static __device__ __forceinline__ void fma(float a, const T &b, float *acc)
    {
        acc[0] = fmaf(a, b.x, acc[0]);
        acc[1] = fmaf(a, b.y, acc[1]);
        acc[2] = fmaf(a, b.z, acc[2]);
        acc[3] = fmaf(a, b.w, acc[3]);
    }
    static __device__ __forceinline__ void store(float *dst, const float *acc)
    {
        *reinterpret_cast<float4 *>(dst) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
};
template <> struct Vec<1> {
    using T = float;
    static __device__ __forceinline__ T zero() { return 0.f; }
    static __device__ __forceinline__ void fma(float a, const T &b, float *acc)
    {
        acc[0] = fmaf(a, b, acc[0]);
    }
    static __device__ __forceinline__ void store(float *dst, const float *acc)
    {
        *dst = acc[0];
    }
};

template <int kLpr, int kVec, bool kVecCsr, bool kOff32>
__global__ __launch_bounds__(kWave) void spmm_kernel(SpmmParams p)
{
    using V = Vec<kVec>;
    using VecT = typename V::T;
    constexpr int kRpw = kWave / kLpr;   // rows per wave
    constexpr int kChunk = 4 * kLpr;     // staged entries per row per window
    constexpr int kPitch = kChunk + 1;   // +1 int2 spreads the groups over banks
    // Staged entry: .x = B-row offset (bytes if kOff32, else the column), .y = value bits.
    __shared__ int2 s_ent[kRpw * kPitch];

    const int lane = threadIdx.x;
    const int grp = lane / kLpr;
    const int gl = lane - grp * kLpr;
    const int tile = blockIdx.x / p.row_blocks;
    const int rb = blockIdx.x - tile * p.row_blocks;
    const long long z = blockIdx.y;
    const float *__restrict__ vals = p.values + z * p.stride_values;
    const float *__restrict__ bz = p.b + z * p.stride_b;
    float *__restrict__ cz = p.c + z * p.stride_c;

    const int slot = rb * kRpw + grp;
    const bool has_row = slot < p.m;
    const int row = has_row ? (p.row_indices ? p.row_indices[slot] : slot) : 0;
    const int p0 = has_row ? p.row_offsets[row] : 0;
    const int p1 = has_row ? p.row_offsets[row + 1] : 0;
    const int col0 = (tile * kLpr + gl) * kVec;
    const bool col_ok = col0 < p.n;  // vector path: n % 4 == 0, so the whole vector is in range
    const unsigned lane_bytes = (unsigned)col0 * 4u;
    int2 *ent = s_ent + grp * kPitch;

    auto offset_of = [&](int col) -> int {
        if constexpr (kOff32)
            return (int)((unsigned)col * (unsigned)p.n * 4u);
        else
            return col;
    };
    auto load_b = [&](int off) -> VecT {
        if constexpr (kOff32)
            return *reinterpret_cast<const VecT *>(
                reinterpret_cast<const char *>(bz) + ((unsigned)off + lane_bytes));
        else
            return *reinterpret_cast<const VecT *>(bz + (size_t)off * (size_t)p.n + col0);
    };

    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;

    int win = kVecCsr ? (p0 & ~3) : p0;
    for (;;) {
        const bool more = win < p1;
        if (!__any(more)) break;  // wave-uniform: every lane reaches the barriers
        if (more) {
            if constexpr (kVecCsr) {
                const int e = win + gl * 4;
                int cc[4];
                float vv[4];
                if (e + 4 <= p.nnz) {
                    const int4 c4 = *reinterpret_cast<const int4 *>(p.col_indices + e);
                    const float4 v4 = *reinterpret_cast<const float4 *>(vals + e);
                    cc[0] = c4.x; cc[1] = c4.y; cc[2] = c4.z; cc[3] = c4.w;
                    vv[0] = v4.x; vv[1] = v4.y; vv[2] = v4.z; vv[3] = v4.w;
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const bool in = e + t < p.nnz;
                        cc[t] = in ? p.col_indices[e + t] : 0;
                        vv[t] = in ? vals[e + t] : 0.f;
                    }
                }
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    ent[gl * 4 + t] = make_int2(offset_of(cc[t]), __float_as_int(vv[t]));
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int idx = win + t * kLpr + gl;
                    const bool in = idx < p1;
                    const int cc = in ? p.col_indices[idx] : 0;
                    const float vv = in ? vals[idx] : 0.f;
                    ent[t * kLpr + gl] = make_int2(offset_of(cc), __float_as_int(vv));
                }
            }
        }
        __syncthreads();
        if (more && col_ok) {
            const int jb = max(p0 - win, 0);  // > 0 only for a misaligned first window
            const int je = min(p1 - win, kChunk);
            int j = jb;
            for (; j + kSpmmUnroll <= je; j += kSpmmUnroll) {
                int2 en[kSpmmUnroll];
                VecT bv[kSpmmUnroll];
#pragma unroll
                for (int u = 0; u < kSpmmUnroll; ++u) en[u] = ent[j + u];
#pragma unroll
                for (int u = 0; u < kSpmmUnroll; ++u) bv[u] = load_b(en[u].x);
#pragma unroll
                for (int u = 0; u < kSpmmUnroll; ++u) V::fma(__int_as_float(en[u].y), bv[u], acc);
            }
            for (; j < je; ++j) {
                const int2 en = ent[j];
                V::fma(__int_as_float(en.y), load_b(en.x), acc);
            }
        }
        __syncthreads();
        win += kChunk;
    }
    if (has_row && col_ok) V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
}

template <int kLpr, int kVec, bool kVecCsr, bool kOff32>
hipError_t launch_t(const SpmmParams &p, int tiles, int batch, hipStream_t s)
{
    dim3 grid((unsigned)(tiles * p.row_blocks), (unsigned)batch);
    hipLaunchKernelGGL((spmm_kernel<kLpr, kVec, kVecCsr, kOff32>), grid,
                       dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <int kLpr, int kVec>
hipError_t launch_csr(const SpmmParams &p, int tiles, int batch, bool vec_csr,
                      bool off32, hipStream_t s)
{
    if (vec_csr)
        return off32 ? launch_t<kLpr, kVec, true, true>(p, tiles, batch, s)
                     : launch_t<kLpr, kVec, true, false>(p, tiles, batch, s);
    return off32 ? launch_t<kLpr, kVec, false, true>(p, tiles, batch, s)
                 : launch_t<kLpr, kVec, false, false>(p, tiles, batch, s);
}

template <int kVec>
hipError_t launch_lpr(int lpr, const SpmmParams &p, int tiles, int batch,
                      bool vec_csr, bool off32, hipStream_t s)
{
    switch (lpr) {
    case 8: return launch_csr<8, kVec>(p, tiles, batch, vec_csr, off32, s);
    case 16: return launch_csr<16, kVec>(p, tiles, batch, vec_csr, off32, s);
    case 32: return launch_csr<32, kVec>(p, tiles, batch, vec_csr, off32, s);
    default: return launch_csr<64, kVec>(p, tiles, batch, vec_csr, off32, s);
    }
}

inline bool aligned16(const void *ptr)
{
    return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0;
}

}  // namespace

// Lanes per row: the smallest of 8/16/32/64 that covers the row's vectors,
// else 64 with several column tiles.  A grid that would not fit the launch
// limits returns hipErrorInvalidConfiguration without launching.
hipError_t launch_spmm(const SpmmArgs &a, hipStream_t stream)
{
    const bool vec = (a.n % 4 == 0) && aligned16(a.b) && aligned16(a.c) &&
                     (a.stride_b % 4 == 0) && (a.stride_c % 4 == 0);
    const bool vec_csr = aligned16(a.col_indices) && aligned16(a.values) &&
                         (a.stride_values % 4 == 0);
    const bool off32 = (long long)a.k * (long long)a.n < (1LL << 30);
    const int kvec = vec ? 4 : 1;
    const int nv = (a.n + kvec - 1) / kvec;
    const int lpr = nv <= 8 ? 8 : nv <= 16 ? 16 : nv <= 32 ? 32 : 64;
    const int rpw = kWave / lpr;
    const int tiles = (nv + lpr - 1) / lpr;
    const long long row_blocks = ((long long)a.m + rpw - 1) / rpw;
    if ((long long)tiles * row_blocks > 0x7fffffffLL || a.batch > 65535)
        return hipErrorInvalidConfiguration;

    SpmmParams p;
    p.m = a.m;
    p.n = a.n;
    p.nnz = a.nnz;
    p.row_blocks = (int)row_blocks;
    p.row_indices = a.row_indices;
    p.row_offsets = a.row_offsets;
    p.col_indices = a.col_indices;
    p.values = a.values;
    p.b = a.b;
    p.c = a.c;
    p.stride_values = a.stride_values;
    p.stride_b = a.stride_b;
    p.stride_c = a.stride_c;
    return vec ? launch_lpr<4>(lpr, p, tiles, a.batch, vec_csr, off32, stream)
               : launch_lpr<1>(lpr, p, tiles, a.batch, vec_csr, off32, stream);
}

}  // namespace spk

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
// Staging.  A group copies its row's (B-row offset, value) pairs into LDS one
// window of kEpl * kLpr entries at a time.  On the vector path each lane reads
// 16-byte segments of col_indices and values with dwordx4 loads, starting from
// the row's first entry rounded down to a multiple of 4; slots before the
// row's start (the misaligned prefix) or after its end become padding.  A
// segment that holds no entry of the row is not loaded.
//
// Gathers.  B is read through a buffer resource: a padding slot carries an
// offset beyond the resource's range, for which the hardware returns zeros
// without touching memory, and its value is 0.  Every gather is therefore
// unconditional, batches of kU gathers are issued back to back, and the next
// batch is in flight while the current one is summed (two register buffers).
// Loop bounds are wave-uniform: a group whose row is done reads padding, so
// multi-row waves never diverge.  B larger than 2 GiB takes the same kernel
// with 64-bit addresses and per-slot predicates instead.
//
// Order of summation: entries of a row in CSR order, sequentially, with fused
// multiply-add (a padding slot adds 0 * 0) -- deterministic, and identical
// whatever row order is used.
#include "sp_device.h"
#include "sp_launch.h"

namespace spk {

namespace {

#ifndef SP_SPMM_UNROLL
#define SP_SPMM_UNROLL 4
#endif
#ifndef SP_SPMM_ENTRIES_PER_LANE
#define SP_SPMM_ENTRIES_PER_LANE 8
#endif
constexpr int kU = SP_SPMM_UNROLL;                // gathers per batch
constexpr int kEpl = SP_SPMM_ENTRIES_PER_LANE;    // staged entries per lane per window
constexpr unsigned kOutOfRange = 0x80000000u;     // buffer offset that reads as zero
static_assert(kEpl % 4 == 0, "segments of 4 entries");

struct SpmmParams {
    int m, n, nnz, row_blocks, tiles, batch;
    unsigned b_bytes;    // bytes of one B operand (buffer path)
    unsigned csr_bytes;  // bytes of col_indices (= of one values array), narrow kernel
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
    static __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
        return make_float4(__uint_as_float(v[0]), __uint_as_float(v[1]),
                           __uint_as_float(v[2]), __uint_as_float(v[3]));
    }
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
    static __device__ __forceinline__ T buf_load(__amdgpu_buffer_rsrc_t r, unsigned off)
    {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
    static __device__ __forceinline__ void fma(float a, const T &b, float *acc)
    {
        acc[0] = fmaf(a, b, acc[0]);
    }
    static __device__ __forceinline__ void store(float *dst, const float *acc)
    {
        *dst = acc[0];
    }
};

// kBuf: B < 2 GiB, gathers through a buffer resource with byte offsets.
// Otherwise: 64-bit addressing, staged offsets are columns, padding has value
// 0 and column -1 and is skipped by a predicate.
template <int kLpr, int kVec, bool kVecCsr, bool kBuf>
__global__ __launch_bounds__(kWave) void spmm_kernel(SpmmParams p)
{
    using V = Vec<kVec>;
    using VecT = typename V::T;
    constexpr int kRpw = kWave / kLpr;       // rows per wave
    constexpr int kChunk = kEpl * kLpr;      // entries per row per window
    // A group's slots: the window, kU padding slots read by the prefetch, and
    // 4 more so that the groups' regions start 12 words apart modulo the 64
    // LDS banks (their broadcast reads then never share a bank).
    constexpr int kPitch = kChunk + kU + 4;
    constexpr int kPad = kBuf ? (int)kOutOfRange : -1;
    static_assert(kPitch % 4 == 0 && kU % 4 == 0, "16-byte aligned batches");
    static_assert(kChunk % kU == 0, "batches never straddle the window end");
    // Staged entries, one array per field so that each lane's staging writes
    // are 16 contiguous bytes: B-row byte offset (kBuf) or column, and value.
    __shared__ __align__(16) int s_off[kRpw * kPitch];
    __shared__ __align__(16) float s_val[kRpw * kPitch];

    const long long w = xcd_work_index((long long)p.batch * p.tiles, p.row_blocks);
    if (w < 0) return;
    const long long per_z = (long long)p.tiles * p.row_blocks;
    const long long z = w / per_z;
    const int tile = (int)((w - z * per_z) / p.row_blocks);
    const int rb = (int)(w - z * per_z - (long long)tile * p.row_blocks);

    const int lane = threadIdx.x;
    const int grp = kRpw == 1 ? 0 : lane / kLpr;
    const int gl = kRpw == 1 ? lane : lane - grp * kLpr;
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
    // Lanes past the last column read only out-of-range (zero) data.
    const unsigned lane_bytes = col_ok ? (unsigned)col0 * 4u : kOutOfRange;
    int *g_off = s_off + grp * kPitch;
    float *g_val = s_val + grp * kPitch;
    for (int j = gl; j < kU; j += kLpr) {
        g_off[kChunk + j] = kPad;
        g_val[kChunk + j] = 0.f;
    }

    __amdgpu_buffer_rsrc_t rsrc;
    if constexpr (kBuf)
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(bz), 0, p.b_bytes,
                                                 0x00020000);

    auto offset_of = [&](int idx, int col) -> int {
        const bool in = idx >= p0 && idx < p1;
        if constexpr (kBuf)
            return in ? (int)((unsigned)col * (unsigned)p.n * 4u) : kPad;
        else
            return in ? col : kPad;
    };
    auto value_of = [&](int idx, float v) -> float {
        return (idx >= p0 && idx < p1) ? v : 0.f;
    };
    auto gather = [&](int off) -> VecT {
        if constexpr (kBuf) {
            return V::buf_load(rsrc, (unsigned)off + lane_bytes);
        } else {
            if (off < 0 || !col_ok) return V::zero();
            return *reinterpret_cast<const VecT *>(bz + (size_t)off * (size_t)p.n + col0);
        }
    };
    // kU staged entries starting at slot j (a multiple of 4): 16-byte
    // broadcast reads of both arrays.
    auto read_batch = [&](int j, int (&off)[kU], float (&val)[kU]) {
#pragma unroll
        for (int u = 0; u < kU; u += 4) {
            const int4 o4 = *reinterpret_cast<const int4 *>(g_off + j + u);
            const float4 v4 = *reinterpret_cast<const float4 *>(g_val + j + u);
            off[u] = o4.x; off[u + 1] = o4.y; off[u + 2] = o4.z; off[u + 3] = o4.w;
            val[u] = v4.x; val[u + 1] = v4.y; val[u + 2] = v4.z; val[u + 3] = v4.w;
        }
    };

    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;

    int win = kVecCsr ? (p0 & ~3) : p0;
    for (;;) {
        const bool more = win < p1;
        if (!__any(more)) break;  // wave-uniform: every lane reaches the barriers
        // ---- stage one window (padding outside [p0, p1))
        if constexpr (kVecCsr) {
#pragma unroll
            for (int sg = 0; sg < kEpl / 4; ++sg) {
                const int slot0 = (sg * kLpr + gl) * 4;
                const int e = win + slot0;
                int cc[4] = {0, 0, 0, 0};
                float vv[4] = {0.f, 0.f, 0.f, 0.f};
                if (e < p1 && e + 4 > p0) {
                    if (e + 4 <= p.nnz) {
                        const int4 c4 = *reinterpret_cast<const int4 *>(p.col_indices + e);
                        const float4 v4 = *reinterpret_cast<const float4 *>(vals + e);
                        cc[0] = c4.x; cc[1] = c4.y; cc[2] = c4.z; cc[3] = c4.w;
                        vv[0] = v4.x; vv[1] = v4.y; vv[2] = v4.z; vv[3] = v4.w;
                    } else {
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            if (e + t < p.nnz) {
                                cc[t] = p.col_indices[e + t];
                                vv[t] = vals[e + t];
                            }
                        }
                    }
                }
                *reinterpret_cast<int4 *>(g_off + slot0) =
                    make_int4(offset_of(e, cc[0]), offset_of(e + 1, cc[1]),
                              offset_of(e + 2, cc[2]), offset_of(e + 3, cc[3]));
                *reinterpret_cast<float4 *>(g_val + slot0) =
                    make_float4(value_of(e, vv[0]), value_of(e + 1, vv[1]),
                                value_of(e + 2, vv[2]), value_of(e + 3, vv[3]));
            }
        } else {
#pragma unroll
            for (int t = 0; t < kEpl; ++t) {
                const int idx = win + t * kLpr + gl;
                const bool in = idx < p1;
                g_off[t * kLpr + gl] = offset_of(idx, in ? p.col_indices[idx] : 0);
                g_val[t * kLpr + gl] = value_of(idx, in ? vals[idx] : 0.f);
            }
        }
        __syncthreads();
        // ---- gather and accumulate: double-buffered batches of kU slots.
        // Slots [0, wend) of the window cover every group's live entries.
        const int my_end = min(p1 - win, kChunk);
        int wend = my_end;
#pragma unroll
        for (int o = kLpr; o < kWave; o <<= 1) wend = max(wend, __shfl_xor(wend, o));
        VecT bufa[kU], bufb[kU];
        int offa[kU], offb[kU];
        float vala[kU], valb[kU];
        // Each batch's staged entries are read right after the arithmetic
        // that frees their registers, and the loop body is one basic block
        // (two batches per trip, the second possibly all padding): the
        // compiler's wait counts are then exact and the next batch's gathers
        // are issued before the current batch is waited for.  Batches past
        // the window are the kU padding slots (min(., kChunk)).
        read_batch(0, offa, vala);
#pragma unroll
        for (int u = 0; u < kU; ++u) bufa[u] = gather(offa[u]);
        read_batch(min(kU, kChunk), offb, valb);
        int j = 0;
        do {
#pragma unroll
            for (int u = 0; u < kU; ++u) bufb[u] = gather(offb[u]);
            keep_issued_above();
#pragma unroll
            for (int u = 0; u < kU; ++u) V::fma(vala[u], bufa[u], acc);
            read_batch(min(j + 2 * kU, kChunk), offa, vala);
#pragma unroll
            for (int u = 0; u < kU; ++u) bufa[u] = gather(offa[u]);
            keep_issued_above();
#pragma unroll
            for (int u = 0; u < kU; ++u) V::fma(valb[u], bufb[u], acc);
            read_batch(min(j + 3 * kU, kChunk), offb, valb);
            j += 2 * kU;
        } while (j < wend);
        __syncthreads();
        win += kChunk;
    }
    if (has_row && col_ok) V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
}

// Narrow B (n of at most 16 columns): the lane-over-columns mapping above
// would leave most of a row group idle, so here the lanes of one wave split
// a row's entries instead.  Lane (s, v) handles entries s, s + kS, s + 2kS, ...
// of the row (kS = 64 / kE entry slots) and the v-th vector of kVec columns
// of B (kE vectors cover the row of B).  Column indices and values are read
// through buffer resources (out-of-range past the row's end: zeros, no
// traffic); each lane sums its entries in order, then the kS partial sums of
// each column vector are added by a shuffle tree over the lane bits above kE.
// Deterministic; a different (tree) order from the wide kernel.
template <int kE, int kVec>
__global__ __launch_bounds__(kWave) void spmm_narrow_kernel(SpmmParams p)
{
    using V = Vec<kVec>;
    using VecT = typename V::T;
    constexpr int kS = kWave / kE;  // entries per step
    constexpr int kSteps = 8;       // steps per batch (CSR loads, then gathers)
    const long long w = xcd_work_index(p.batch, p.m);
    if (w < 0) return;
    const long long z = w / p.m;
    const int slot = (int)(w - z * p.m);
    const int lane = threadIdx.x;
    const int s = lane / kE;
    const int v = lane - s * kE;
    const int row = p.row_indices ? p.row_indices[slot] : slot;
    const int p0 = p.row_offsets[row];
    const int p1 = p.row_offsets[row + 1];
    const float *vals = p.values + z * p.stride_values;
    const float *bz = p.b + z * p.stride_b;
    float *cz = p.c + z * p.stride_c;
    const int col0 = v * kVec;
    const bool col_ok = col0 < p.n;
    const unsigned lane_bytes = col_ok ? (unsigned)col0 * 4u : kOutOfRange;
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(bz), 0, (int)p.b_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int *>(p.col_indices), 0, (int)p.csr_bytes, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float *>(vals), 0, (int)p.csr_bytes, 0x00020000);

    float acc[kVec];
#pragma unroll
    for (int t = 0; t < kVec; ++t) acc[t] = 0.f;
    for (int base = p0; base < p1; base += kS * kSteps) {  // wave-uniform bound
        unsigned coff[kSteps];
        int cc[kSteps];
        float vv[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const int idx = base + u * kS + s;
            coff[u] = idx < p1 ? (unsigned)idx * 4u : kOutOfRange;
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            cc[u] = (int)__builtin_amdgcn_raw_buffer_load_b32(rc, (int)coff[u], 0, 0);
            vv[u] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rv, (int)coff[u], 0, 0));
        }
        VecT bv[kSteps];
#pragma unroll
        for (int u = 0; u < kSteps; ++u) {
            const unsigned off = coff[u] == kOutOfRange
                                     ? kOutOfRange
                                     : (unsigned)cc[u] * (unsigned)p.n * 4u + lane_bytes;
            bv[u] = V::buf_load(rb, off);
        }
#pragma unroll
        for (int u = 0; u < kSteps; ++u) V::fma(vv[u], bv[u], acc);
    }
#pragma unroll
    for (int o = kE; o < kWave; o <<= 1) {
#pragma unroll
        for (int t = 0; t < kVec; ++t) acc[t] += __shfl_xor(acc[t], o);
    }
    if (s == 0 && col_ok) V::store(cz + (size_t)row * (size_t)p.n + col0, acc);
}

template <int kE, int kVec>
hipError_t launch_narrow_t(const SpmmParams &p, hipStream_t s)
{
    dim3 grid((unsigned)xcd_grid(p.batch, p.m));
    hipLaunchKernelGGL((spmm_narrow_kernel<kE, kVec>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <int kVec>
hipError_t launch_narrow(int e, const SpmmParams &p, hipStream_t s)
{
    switch (e) {
    case 1: return launch_narrow_t<1, kVec>(p, s);
    case 2: return launch_narrow_t<2, kVec>(p, s);
    default: return launch_narrow_t<4, kVec>(p, s);
    }
}

template <int kLpr, int kVec, bool kVecCsr, bool kBuf>
hipError_t launch_t(const SpmmParams &p, int tiles, int batch, hipStream_t s)
{
    (void)tiles;
    (void)batch;
    dim3 grid((unsigned)xcd_grid((long long)p.batch * p.tiles, p.row_blocks));
    hipLaunchKernelGGL((spmm_kernel<kLpr, kVec, kVecCsr, kBuf>), grid, dim3(kWave), 0, s, p);
    return hipGetLastError();
}

template <int kLpr, int kVec>
hipError_t launch_csr(const SpmmParams &p, int tiles, int batch, bool vec_csr, bool buf,
                      hipStream_t s)
{
    if (vec_csr)
        return buf ? launch_t<kLpr, kVec, true, true>(p, tiles, batch, s)
                   : launch_t<kLpr, kVec, true, false>(p, tiles, batch, s);
    return buf ? launch_t<kLpr, kVec, false, true>(p, tiles, batch, s)
               : launch_t<kLpr, kVec, false, false>(p, tiles, batch, s);
}

template <int kVec>
hipError_t launch_lpr(int lpr, const SpmmParams &p, int tiles, int batch, bool vec_csr,
                      bool buf, hipStream_t s)
{
    switch (lpr) {
    case 8: return launch_csr<8, kVec>(p, tiles, batch, vec_csr, buf, s);
    case 16: return launch_csr<16, kVec>(p, tiles, batch, vec_csr, buf, s);
    case 32: return launch_csr<32, kVec>(p, tiles, batch, vec_csr, buf, s);
    default: return launch_csr<64, kVec>(p, tiles, batch, vec_csr, buf, s);
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
    // Valid offsets stay below B's size and padding offsets (>= 2^31) beyond it.
    const bool buf = (long long)a.k * (long long)a.n <= (1LL << 29);
    const int kvec = vec ? 4 : 1;
    const int nv = (a.n + kvec - 1) / kvec;
    const int lpr = nv <= 8 ? 8 : nv <= 16 ? 16 : nv <= 32 ? 32 : 64;
    const int rpw = kWave / lpr;
    const int tiles = (nv + lpr - 1) / lpr;
    const long long row_blocks = ((long long)a.m + rpw - 1) / rpw;
    if (xcd_grid((long long)a.batch * tiles, row_blocks) > 0x7fffffffLL)
        return hipErrorInvalidConfiguration;

    // Narrow B: lanes over entries (needs the buffer paths for B and the CSR).
    const bool narrow = buf && nv <= 4 && (long long)a.nnz * 4 <= (1LL << 31);
    if (narrow && xcd_grid(a.batch, a.m) > 0x7fffffffLL) return hipErrorInvalidConfiguration;

    SpmmParams p;
    p.m = a.m;
    p.n = a.n;
    p.nnz = a.nnz;
    p.row_blocks = (int)row_blocks;
    p.tiles = tiles;
    p.batch = a.batch;
    p.b_bytes = buf ? (unsigned)((long long)a.k * a.n * 4) : 0u;
    p.csr_bytes = narrow ? (unsigned)((long long)a.nnz * 4) : 0u;
    p.row_indices = a.row_indices;
    p.row_offsets = a.row_offsets;
    p.col_indices = a.col_indices;
    p.values = a.values;
    p.b = a.b;
    p.c = a.c;
    p.stride_values = a.stride_values;
    p.stride_b = a.stride_b;
    p.stride_c = a.stride_c;
    if (narrow) {
        const int e = nv <= 1 ? 1 : nv <= 2 ? 2 : 4;
        return vec ? launch_narrow<4>(e, p, stream) : launch_narrow<1>(e, p, stream);
    }
    return vec ? launch_lpr<4>(lpr, p, tiles, a.batch, vec_csr, buf, stream)
               : launch_lpr<1>(lpr, p, tiles, a.batch, vec_csr, buf, stream);
}

}  // namespace spk

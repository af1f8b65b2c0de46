// mr.hip -- dense NN search and reciprocal matching for MI355X (gfx950, CDNA4).
//
// One similarity/argmax kernel serves every entry point: a block of queries
// (gathered rows of one map, held in registers as the MFMA B operand) against
// a contiguous range of rows of the other map (streamed as the MFMA A
// operand), d-component contraction on the matrix cores, a running per-lane
// (score, row) maximum with the lowest row winning ties, and a 64-bit atomic
// max on packed (ordered score, ~row) keys to merge database ranges.  The
// similarity matrix never leaves registers.
//
// The maths, cited by page title and section:
//  - s(i, j) = <D1[i], D2[j]>, NN = argmax ("MASt3R dissection", section 3
//    "Napkin Formula"); reciprocal pairs are mutual NNs (same page, section 1
//    diagram).
//  - Fast reciprocal matching: seeds on a sparse grid, forward and backward NN,
//    keep cycle-consistent pairs, restart the rest where they landed ("DUSt3R
//    and MASt3R explained", the paragraph on MASt3R's fast reciprocal
//    matching).
//
// Layout of the MFMA operands (wave64, 16x16 output tile):
//  - lane l holds output column j = l & 15 (a query) and rows
//    i = 4*(l >> 4) + v, v = 0..3 (four database rows) of every tile;
//  - fp32 maps use V_MFMA_F32_16X16X4_F32 in P = ceil(d/4) steps; in step s
//    lane group g = l >> 4 supplies component c = P*g + s of its row;
//  - bf16 maps use V_MFMA_F32_16X16X32_BF16 in P = ceil(d/32) steps; in step s
//    lane group g supplies components 8*(P*g + s) .. +7 (zero past d).
// A and B use the same component-to-k assignment, products commute, and the
// accumulation order depends only on k, so s(i, j) is bitwise identical
// whichever map is the query side.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "mr.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = 8;           // 16-query tiles held per wave
constexpr int kQBW = 16 * kQT;   // queries per wave
constexpr int kCompactChunk = 2048;  // elements per block in the ordered compaction
constexpr int kMaxD = 64;
constexpr int kTargetWaves = 4096;   // 256 CUs x 4 SIMDs x 4 waves

// ---------------------------------------------------------------------------- keys

// Order-preserving map of an fp32 score to uint32 (+0 and -0 map alike).
__device__ __forceinline__ uint32_t ordered_bits(float s) {
    uint32_t u = __float_as_uint(s);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float from_ordered(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Larger key = higher score, then lower row.  0 = "no candidate".
__device__ __forceinline__ uint64_t pack_key(float s, uint32_t row) {
    return ((uint64_t)ordered_bits(s) << 32) | (uint64_t)(~row);
}

__device__ __forceinline__ int32_t key_row(uint64_t k) {
    return k ? (int32_t)(~(uint32_t)k) : -1;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    uint32_t lo = __shfl_xor((uint32_t)x, m);
    uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------- operands

template <int DT, int P> struct Operand;

template <int P> struct Operand<MR_F32, P> {
    float x[P];
    __device__ __forceinline__ void load(const void* base, int64_t row, bool valid, int g, int d) {
        // branch-free: out-of-range components read the row's first element, then select 0
        const float* p = static_cast<const float*>(base) + row * d;
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int c = P * g + s;
            const bool ok = valid && c < d;
            const float t = p[ok ? c : 0];
            x[s] = ok ? t : 0.0f;
        }
    }
    __device__ __forceinline__ f32x4 mfma(const Operand& b, f32x4 acc) const {
#pragma unroll
        for (int s = 0; s < P; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(x[s], b.x[s], acc, 0, 0, 0);
        return acc;
    }
};

template <int P> struct Operand<MR_BF16, P> {
    bf16x8 x[P];
    __device__ __forceinline__ void load(const void* base, int64_t row, bool valid, int g, int d) {
        const uint16_t* p = static_cast<const uint16_t*>(base) + row * d;
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int c = 8 * (P * g + s);
            const bool ok = valid && c < d;
            u32x4 raw = *reinterpret_cast<const u32x4*>(p + (ok ? c : 0));
            if (!ok) raw = u32x4{0u, 0u, 0u, 0u};
            x[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    __device__ __forceinline__ f32x4 mfma(const Operand& b, f32x4 acc) const {
#pragma unroll
        for (int s = 0; s < P; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(x[s], b.x[s], acc, 0, 0, 0);
        return acc;
    }
};

// ---------------------------------------------------------------------------- NN kernel

enum QuerySource { Q_ALL = 0, Q_LIST = 1, Q_KEYS = 2 };

struct NNArgs {
    const void* qmap;        // [batch][nq_rows][d]
    const void* dbmap;       // [batch][ndb][d]
    int64_t q_pair_elems;    // nq_rows * d
    int64_t db_pair_elems;   // ndb * d
    int32_t nq_rows;
    int32_t ndb;
    int32_t d;
    int32_t qsrc;            // QuerySource
    const void* qlist;       // int32 rows (Q_LIST) or uint64 keys (Q_KEYS), [batch][qlist_stride]
    int64_t qlist_stride;
    const int32_t* dev_count;  // per-pair query count on the device, or NULL
    int64_t count_stride;
    int32_t host_count;        // query count when dev_count is NULL
    uint64_t* keys;            // [batch][keys_stride] results, merged with atomicMax
    int64_t keys_stride;
    int32_t* active_out;       // optional: record the query count here (per pair)
    int64_t active_stride;
    int32_t* zero_count;       // optional: set this per-pair counter to 0
    int64_t zero_stride;
};

// Each wave owns (query block, database segment) work items; the number of
// segments adapts to the live query count so small frontiers still fill the GPU.
template <int DT, int P>
__global__ __launch_bounds__(kThreads) void nn_argmax_kernel(NNArgs a) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int jl = lane & 15;
    const int pair = blockIdx.y;
    const int n = a.dev_count ? a.dev_count[pair * a.count_stride] : a.host_count;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        if (a.active_out) a.active_out[pair * a.active_stride] = n;
        if (a.zero_count) a.zero_count[pair * a.zero_stride] = 0;
    }
    const int ntiles = (a.ndb + 15) >> 4;
    const int qblocks = (n + kQBW - 1) / kQBW;
    if (qblocks == 0 || ntiles == 0) return;
    const int total_waves = gridDim.x * kWaves;
    int nseg = total_waves / qblocks;
    nseg = nseg < 1 ? 1 : (nseg > ntiles ? ntiles : nseg);
    const int items = qblocks * nseg;
    const int full_tiles = a.ndb >> 4;

    const void* qbase = (DT == MR_F32)
        ? (const void*)(static_cast<const float*>(a.qmap) + pair * a.q_pair_elems)
        : (const void*)(static_cast<const uint16_t*>(a.qmap) + pair * a.q_pair_elems);
    const void* dbase = (DT == MR_F32)
        ? (const void*)(static_cast<const float*>(a.dbmap) + pair * a.db_pair_elems)
        : (const void*)(static_cast<const uint16_t*>(a.dbmap) + pair * a.db_pair_elems);

    for (int it = blockIdx.x * kWaves + (threadIdx.x >> 6); it < items; it += total_waves) {
        const int seg = it / qblocks;
        const int qb = it - seg * qblocks;

        // queries of this block -> B operands
        Operand<DT, P> q[kQT];
#pragma unroll
        for (int j = 0; j < kQT; ++j) {
            const int qp = qb * kQBW + j * 16 + jl;
            int64_t row = qp;
            bool valid = qp < n;
            if (valid && a.qsrc == Q_LIST)
                row = static_cast<const int32_t*>(a.qlist)[pair * a.qlist_stride + qp];
            else if (valid && a.qsrc == Q_KEYS)
                row = key_row(static_cast<const uint64_t*>(a.qlist)[pair * a.qlist_stride + qp]);
            valid = valid && row >= 0 && row < a.nq_rows;
            q[j].load(qbase, valid ? row : 0, valid, g, a.d);
        }

        const int t0 = (int)((int64_t)seg * ntiles / nseg);
        const int t1 = (int)((int64_t)(seg + 1) * ntiles / nseg);
        const int tf = t1 < full_tiles ? t1 : full_tiles;

        float bv[kQT];
        int bt[kQT];
#pragma unroll
        for (int j = 0; j < kQT; ++j) { bv[j] = -INFINITY; bt[j] = -1; }

        // full tiles: every row valid
        for (int t = t0; t < tf; ++t) {
            Operand<DT, P> r;
            r.load(dbase, (int64_t)t * 16 + jl, true, g, a.d);
#pragma unroll
            for (int j = 0; j < kQT; ++j) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = r.mfma(q[j], acc);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float s = acc[v];
                    const bool gt = s > bv[j];
                    bv[j] = gt ? s : bv[j];
                    bt[j] = gt ? (t * 4 + v) : bt[j];
                }
            }
        }
        // the ragged last tile
        if (tf < t1) {
            const int t = tf;
            const int64_t rrow = (int64_t)t * 16 + jl;
            Operand<DT, P> r;
            r.load(dbase, rrow < a.ndb ? rrow : 0, rrow < a.ndb, g, a.d);
#pragma unroll
            for (int j = 0; j < kQT; ++j) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                acc = r.mfma(q[j], acc);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const bool ok = t * 16 + 4 * g + v < a.ndb;
                    const float s = acc[v];
                    const bool gt = ok && s > bv[j];
                    bv[j] = gt ? s : bv[j];
                    bt[j] = gt ? (t * 4 + v) : bt[j];
                }
            }
        }

        // merge the four lane groups holding each query, then across segments
#pragma unroll
        for (int j = 0; j < kQT; ++j) {
            uint64_t key = 0;
            if (bt[j] >= 0) {
                const uint32_t row = (uint32_t)((bt[j] >> 2) * 16 + 4 * g + (bt[j] & 3));
                key = pack_key(bv[j], row);
            }
            uint64_t o = shfl_xor_u64(key, 16);
            key = o > key ? o : key;
            o = shfl_xor_u64(key, 32);
            key = o > key ? o : key;
            const int qp = qb * kQBW + j * 16 + jl;
            if (g == 0 && qp < n && key != 0)
                atomicMax(reinterpret_cast<unsigned long long*>(&a.keys[pair * a.keys_stride + qp]),
                          (unsigned long long)key);
        }
    }
}

// ---------------------------------------------------------------------------- small kernels

__global__ void fill_u64_kernel(uint64_t* p, int64_t n, uint64_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// keys -> row ids (and optionally scores)
__global__ void decode_keys_kernel(const uint64_t* keys, int64_t n, int32_t* idx, float* score) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t k = keys[i];
        idx[i] = key_row(k);
        if (score) score[i] = k ? from_ordered((uint32_t)(k >> 32)) : -INFINITY;
    }
}

// Fast scheme set-up: per pixel of image a, state = -2 for seeds (live), -1 otherwise;
// seed k (row-major on the grid) goes to frontier slot k; counters and round-0 keys reset.
struct InitArgs {
    int32_t* state; int64_t n1; int32_t w;
    int32_t stride, offset, nx, nseeds;
    int32_t* front0; uint64_t* keys_f0; uint64_t* keys_b0; int64_t slot_stride;
    int32_t* cnt0; int32_t* cnt1;
};

__global__ void fast_init_kernel(InitArgs a) {
    const int pair = blockIdx.y;
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < a.n1;
         p += (int64_t)gridDim.x * blockDim.x) {
        const int32_t y = (int32_t)(p / a.w), x = (int32_t)(p - (int64_t)y * a.w);
        const bool seed = y >= a.offset && x >= a.offset && (y - a.offset) % a.stride == 0 &&
                          (x - a.offset) % a.stride == 0;
        a.state[pair * a.n1 + p] = seed ? -2 : -1;
        if (seed) {
            const int64_t k = (int64_t)((y - a.offset) / a.stride) * a.nx + (x - a.offset) / a.stride;
            a.front0[pair * a.slot_stride + k] = (int32_t)p;
        }
        if (p < a.nseeds) {
            a.keys_f0[pair * a.slot_stride + p] = 0;
            a.keys_b0[pair * a.slot_stride + p] = 0;
        }
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.cnt0[pair] = a.nseeds;
        a.cnt1[pair] = 0;
    }
}

// One reciprocity check per live pixel u: v = NN(a[u], b), u' = NN(b[v], a).
// u' == u: keep (u, v).  Otherwise u' becomes live next iteration if nobody has
// been there (state -1); ballot + prefix sum give each wave one atomic.
struct CycleArgs {
    const int32_t* front; const uint64_t* keys_f; const uint64_t* keys_b;
    uint64_t* keys_f_next; uint64_t* keys_b_next; int32_t* front_next;
    const int32_t* cnt; int32_t* cnt_next; int32_t* state;
    int64_t slot_stride; int64_t n1; int32_t last;
};

__global__ __launch_bounds__(256) void fast_cycle_kernel(CycleArgs a) {
    const int pair = blockIdx.y;
    const int n = a.cnt[pair];
    const int lane = threadIdx.x & 63;
    for (int k0 = blockIdx.x * blockDim.x; k0 < n; k0 += gridDim.x * blockDim.x) {
        const int k = k0 + threadIdx.x;
        bool push = false;
        int32_t u2 = -1;
        if (k < n) {
            const int64_t slot = pair * a.slot_stride + k;
            const int32_t u = a.front[slot];
            const int32_t v = key_row(a.keys_f[slot]);
            u2 = key_row(a.keys_b[slot]);
            a.keys_f_next[slot] = 0;
            a.keys_b_next[slot] = 0;
            if (v >= 0 && u2 >= 0) {
                int32_t* st = a.state + pair * a.n1;
                if (u2 == u) {
                    st[u] = v;
                } else if (!a.last) {
                    push = atomicCAS(&st[u2], -1, -2) == -1;
                }
            }
        }
        const uint64_t mask = __ballot(push);
        if (mask) {
            const int leader = __ffsll((unsigned long long)mask) - 1;
            int at = 0;
            if (lane == leader) at = atomicAdd(&a.cnt_next[pair], (int)__popcll(mask));
            at = __shfl(at, leader);
            if (push) a.front_next[pair * a.slot_stride + at + __popcll(mask & __lanemask_lt())] = u2;
        }
    }
}

// ---------------------------------------------------------------------------- ordered compaction

// Predicate + payload: element e of pair b is kept as (first, second).
struct FastPred {
    const int32_t* state; int64_t n;
    __device__ __forceinline__ bool get(int pair, int64_t e, int32_t& i, int32_t& j) const {
        const int32_t v = state[pair * n + e];
        i = (int32_t)e; j = v;
        return v >= 0;
    }
};
struct MutualPred {
    const int32_t* nn_ab; const int32_t* nn_ba; int64_t na, nb;
    __device__ __forceinline__ bool get(int pair, int64_t e, int32_t& i, int32_t& j) const {
        const int32_t v = nn_ab[pair * na + e];
        i = (int32_t)e; j = v;
        return v >= 0 && nn_ba[pair * nb + v] == (int32_t)e;
    }
};

template <class Pred>
__global__ __launch_bounds__(256) void compact_count_kernel(Pred pr, int64_t n, int32_t* blk_count, int nblk) {
    __shared__ int wsum[4];
    const int pair = blockIdx.y;
    const int64_t base = (int64_t)blockIdx.x * kCompactChunk;
    int c = 0;
    for (int r = 0; r < kCompactChunk / 256; ++r) {
        const int64_t e = base + r * 256 + threadIdx.x;
        int32_t i, j;
        if (e < n && pr.get(pair, e, i, j)) ++c;
    }
    // wave sum then block sum
    for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m);
    if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) blk_count[pair * nblk + blockIdx.x] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

template <class Pred>
__global__ __launch_bounds__(256) void compact_scatter_kernel(Pred pr, int64_t n, const int32_t* blk_count, int nblk,
                                                              int32_t* pairs, int64_t cap, int64_t* n_pairs) {
    __shared__ int64_t sbase;
    __shared__ int wcnt[4];
    const int pair = blockIdx.y;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    if (wv == 0) {
        int64_t s = 0;
        for (int k = lane; k < (int)blockIdx.x; k += 64) s += blk_count[pair * nblk + k];
        for (int m = 32; m >= 1; m >>= 1) {
            const uint32_t lo = __shfl_xor((uint32_t)s, m), hi = __shfl_xor((uint32_t)((uint64_t)s >> 32), m);
            s += (int64_t)(((uint64_t)hi << 32) | lo);
        }
        if (lane == 0) sbase = s;
    }
    __syncthreads();
    int64_t run = sbase;
    const int64_t base = (int64_t)blockIdx.x * kCompactChunk;
    for (int r = 0; r < kCompactChunk / 256; ++r) {
        const int64_t e = base + r * 256 + threadIdx.x;
        int32_t i = 0, j = 0;
        const bool keep = e < n && pr.get(pair, e, i, j);
        const uint64_t mask = __ballot(keep);
        if (lane == 0) wcnt[wv] = (int)__popcll(mask);
        __syncthreads();
        int off = 0;
        for (int k = 0; k < wv; ++k) off += wcnt[k];
        const int tot = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
        if (keep) {
            const int64_t pos = run + off + __popcll(mask & __lanemask_lt());
            if (pos < cap) {
                pairs[(pair * cap + pos) * 2] = i;
                pairs[(pair * cap + pos) * 2 + 1] = j;
            }
        }
        run += tot;
        __syncthreads();
    }
    if (blockIdx.x == nblk - 1 && threadIdx.x == 0) n_pairs[pair] = run;
}

// ---------------------------------------------------------------------------- host helpers

struct Profiler {
    bool on = false;
    int cap = 0, used = 0;
    hipEvent_t* ev = nullptr;
} g_prof;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

int validate_map(const mr_map* m) {
    if (!m) return MR_ERR_NULL;
    if (m->batch < 1 || m->batch > 65535 || m->h < 0 || m->w < 0 || m->d < 1 || m->d > kMaxD) return MR_ERR_SHAPE;
    if ((int64_t)m->h * m->w > (int64_t(1) << 28)) return MR_ERR_SHAPE;
    if (m->dtype != MR_F32 && m->dtype != MR_BF16) return MR_ERR_DTYPE;
    if (m->dtype == MR_BF16 && (m->d % 8) != 0) return MR_ERR_DTYPE;
    if ((int64_t)m->h * m->w > 0 && !m->data) return MR_ERR_NULL;
    if (m->data && (reinterpret_cast<uintptr_t>(m->data) & 15)) return MR_ERR_SHAPE;
    return MR_OK;
}

int validate_pair(const mr_map* a, const mr_map* b) {
    int rc = validate_map(a);
    if (rc) return rc;
    rc = validate_map(b);
    if (rc) return rc;
    if (a->batch != b->batch || a->d != b->d) return MR_ERR_SHAPE;
    if (a->dtype != b->dtype) return MR_ERR_DTYPE;
    return MR_OK;
}

inline int64_t npix(const mr_map* m) { return (int64_t)m->h * m->w; }
inline int nblk_of(int64_t n) { return (int)((n + kCompactChunk - 1) / kCompactChunk); }

int64_t seed_count(int32_t h, int32_t w, int32_t stride, int32_t offset) {
    if (stride < 1 || offset < 0 || h < 0 || w < 0) return -1;
    const int64_t ny = offset < h ? (h - 1 - offset) / stride + 1 : 0;
    const int64_t nx = offset < w ? (w - 1 - offset) / stride + 1 : 0;
    return ny * nx;
}

int grid_1d(int64_t n, int threads = 256, int cap = 1 << 24) {
    int64_t g = (n + threads - 1) / threads;
    if (g < 1) g = 1;
    return (int)(g > cap ? cap : g);
}

int dev_err() { return hipGetLastError() == hipSuccess ? MR_OK : MR_ERR_DEVICE; }

template <int DT, int P>
void launch_nn_t(const NNArgs& a, dim3 grid, hipStream_t st) {
    hipLaunchKernelGGL((nn_argmax_kernel<DT, P>), grid, dim3(kThreads), 0, st, a);
}

int launch_nn(const NNArgs& a, int dtype, int batch, int gridx, hipStream_t st) {
    const dim3 grid(gridx, batch);
    const bool prof = g_prof.on && g_prof.used < g_prof.cap;
    if (prof && hipEventRecord(g_prof.ev[2 * g_prof.used], st) != hipSuccess) return MR_ERR_DEVICE;
    if (dtype == MR_F32) {
        switch ((a.d + 3) / 4) {
#define MR_CASE(p) case p: launch_nn_t<MR_F32, p>(a, grid, st); break;
            MR_CASE(1) MR_CASE(2) MR_CASE(3) MR_CASE(4) MR_CASE(5) MR_CASE(6) MR_CASE(7) MR_CASE(8)
            MR_CASE(9) MR_CASE(10) MR_CASE(11) MR_CASE(12) MR_CASE(13) MR_CASE(14) MR_CASE(15) MR_CASE(16)
#undef MR_CASE
            default: return MR_ERR_SHAPE;
        }
    } else {
        if (a.d <= 32) launch_nn_t<MR_BF16, 1>(a, grid, st);
        else launch_nn_t<MR_BF16, 2>(a, grid, st);
    }
    if (dev_err()) return MR_ERR_DEVICE;
    if (prof) {
        if (hipEventRecord(g_prof.ev[2 * g_prof.used + 1], st) != hipSuccess) return MR_ERR_DEVICE;
        ++g_prof.used;
    }
    return MR_OK;
}

// Workgroups per pair: enough waves for every (query block, segment) item to fill the GPU.
int nn_grid_x(int64_t n_queries, int batch) {
    const int64_t per_pair = (kTargetWaves + batch - 1) / batch;
    int64_t qblocks = (n_queries + kQBW - 1) / kQBW;
    int64_t waves = per_pair > qblocks ? per_pair : qblocks;
    int64_t wgs = (waves + kWaves - 1) / kWaves;
    if (wgs < 1) wgs = 1;
    return (int)(wgs > 65535 ? 65535 : wgs);
}

NNArgs nn_args(const mr_map* q, const mr_map* db) {
    NNArgs a;
    memset(&a, 0, sizeof(a));
    a.qmap = q->data;
    a.dbmap = db->data;
    a.q_pair_elems = npix(q) * q->d;
    a.db_pair_elems = npix(db) * db->d;
    a.nq_rows = (int32_t)npix(q);
    a.ndb = (int32_t)npix(db);
    a.d = q->d;
    return a;
}

struct FastLayout {
    size_t keys_f[2], keys_b[2], front[2], cnt[2], state, blk, total;
};

FastLayout fast_layout(int batch, int64_t nseeds, int64_t n1) {
    FastLayout L;
    size_t off = 0;
    const size_t slots = (size_t)batch * (size_t)(nseeds > 0 ? nseeds : 1);
    for (int i = 0; i < 2; ++i) { L.keys_f[i] = off; off = align256(off + slots * 8); }
    for (int i = 0; i < 2; ++i) { L.keys_b[i] = off; off = align256(off + slots * 8); }
    for (int i = 0; i < 2; ++i) { L.front[i] = off; off = align256(off + slots * 4); }
    for (int i = 0; i < 2; ++i) { L.cnt[i] = off; off = align256(off + (size_t)batch * 4); }
    L.state = off; off = align256(off + (size_t)batch * (size_t)(n1 > 0 ? n1 : 1) * 4);
    L.blk = off; off = align256(off + (size_t)batch * (size_t)(nblk_of(n1) > 0 ? nblk_of(n1) : 1) * 4);
    L.total = off;
    return L;
}

struct MutualLayout { size_t keys_ab, keys_ba, blk, total; };

MutualLayout mutual_layout(int batch, int64_t na, int64_t nb) {
    MutualLayout L;
    size_t off = 0;
    L.keys_ab = off; off = align256(off + (size_t)batch * (size_t)(na > 0 ? na : 1) * 8);
    L.keys_ba = off; off = align256(off + (size_t)batch * (size_t)(nb > 0 ? nb : 1) * 8);
    L.blk = off; off = align256(off + (size_t)batch * (size_t)(nblk_of(na) > 0 ? nblk_of(na) : 1) * 4);
    L.total = off;
    return L;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (!ws) return MR_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255) return MR_ERR_WORKSPACE;
    if (ws_bytes < need) return MR_ERR_WORKSPACE;
    return MR_OK;
}

template <class T> T* at(void* ws, size_t off) { return reinterpret_cast<T*>(static_cast<char*>(ws) + off); }

}  // namespace

// ============================================================================ C ABI

extern "C" {

const char* mr_status_str(int status) {
    switch (status) {
        case MR_OK: return "ok";
        case MR_ERR_NULL: return "a required pointer is NULL";
        case MR_ERR_SHAPE: return "map sizes out of range or inconsistent";
        case MR_ERR_DTYPE: return "unsupported or mismatched dtype";
        case MR_ERR_PARAM: return "invalid parameter";
        case MR_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MR_ERR_CAPACITY: return "output capacity below the bound";
        case MR_ERR_DEVICE: return "HIP call failed";
        default: return "unknown status";
    }
}

int64_t mr_seed_count(int32_t h, int32_t w, int32_t stride, int32_t offset) {
    return seed_count(h, w, stride, offset);
}

size_t mr_workspace_bytes(int op, const mr_map* a, const mr_map* b, int64_t n_q, int32_t stride,
                          int32_t offset) {
    if (validate_pair(a, b) != MR_OK) return 0;
    switch (op) {
        case MR_OP_NN_ARGMAX:
            if (n_q < 0) return 0;
            return align256((size_t)a->batch * (size_t)(n_q > 0 ? n_q : 1) * 8);
        case MR_OP_MUTUAL_NN:
            return mutual_layout(a->batch, npix(a), npix(b)).total;
        case MR_OP_FAST_RECIPROCAL: {
            const int64_t ns = seed_count(a->h, a->w, stride, offset);
            if (ns < 0) return 0;
            return fast_layout(a->batch, ns, npix(a)).total;
        }
        default: return 0;
    }
}

int mr_nn_argmax(const mr_map* q, const mr_map* db, const int32_t* q_idx, int64_t n_q, int32_t* out_idx,
                 float* out_score, void* ws, size_t ws_bytes, void* stream) {
    int rc = validate_pair(q, db);
    if (rc) return rc;
    if (n_q < 0 || n_q > (int64_t(1) << 28)) return MR_ERR_PARAM;
    if (!q_idx && n_q != npix(q)) return MR_ERR_PARAM;
    if (n_q == 0) return MR_OK;
    if (npix(q) == 0) return MR_ERR_SHAPE;  // query ids cannot name a row of an empty map
    if (!out_idx) return MR_ERR_NULL;
    const size_t need = align256((size_t)q->batch * (size_t)n_q * 8);
    if ((rc = check_ws(ws, ws_bytes, need))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint64_t* keys = static_cast<uint64_t*>(ws);
    const int64_t tot = (int64_t)q->batch * n_q;
    hipLaunchKernelGGL(fill_u64_kernel, dim3(grid_1d(tot)), dim3(256), 0, st, keys, tot, (uint64_t)0);
    if (dev_err()) return MR_ERR_DEVICE;
    NNArgs a = nn_args(q, db);
    a.qsrc = q_idx ? Q_LIST : Q_ALL;
    a.qlist = q_idx;
    a.qlist_stride = n_q;
    a.host_count = (int32_t)n_q;
    a.keys = keys;
    a.keys_stride = n_q;
    if ((rc = launch_nn(a, q->dtype, q->batch, nn_grid_x(n_q, q->batch), st))) return rc;
    hipLaunchKernelGGL(decode_keys_kernel, dim3(grid_1d(tot)), dim3(256), 0, st, keys, tot, out_idx, out_score);
    return dev_err();
}

int mr_mutual_nn(const mr_map* a, const mr_map* b, int32_t* nn_ab, int32_t* nn_ba, int32_t* pairs, int64_t cap,
                 int64_t* n_pairs, void* ws, size_t ws_bytes, void* stream) {
    int rc = validate_pair(a, b);
    if (rc) return rc;
    if (!nn_ab || !nn_ba || !pairs || !n_pairs) return MR_ERR_NULL;
    const int64_t na = npix(a), nb = npix(b);
    const int64_t bound = na < nb ? na : nb;
    if (cap < bound) return MR_ERR_CAPACITY;
    const MutualLayout L = mutual_layout(a->batch, na, nb);
    if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int batch = a->batch;
    uint64_t* kab = at<uint64_t>(ws, L.keys_ab);
    uint64_t* kba = at<uint64_t>(ws, L.keys_ba);
    int32_t* blk = at<int32_t>(ws, L.blk);
    hipLaunchKernelGGL(fill_u64_kernel, dim3(grid_1d(batch * na)), dim3(256), 0, st, kab, batch * na, (uint64_t)0);
    hipLaunchKernelGGL(fill_u64_kernel, dim3(grid_1d(batch * nb)), dim3(256), 0, st, kba, batch * nb, (uint64_t)0);
    if (dev_err()) return MR_ERR_DEVICE;
    NNArgs f = nn_args(a, b);
    f.qsrc = Q_ALL;
    f.host_count = (int32_t)na;
    f.keys = kab;
    f.keys_stride = na;
    if ((rc = launch_nn(f, a->dtype, batch, nn_grid_x(na, batch), st))) return rc;
    NNArgs r = nn_args(b, a);
    r.qsrc = Q_ALL;
    r.host_count = (int32_t)nb;
    r.keys = kba;
    r.keys_stride = nb;
    if ((rc = launch_nn(r, a->dtype, batch, nn_grid_x(nb, batch), st))) return rc;
    hipLaunchKernelGGL(decode_keys_kernel, dim3(grid_1d(batch * na)), dim3(256), 0, st, kab, batch * na, nn_ab,
                       (float*)nullptr);
    hipLaunchKernelGGL(decode_keys_kernel, dim3(grid_1d(batch * nb)), dim3(256), 0, st, kba, batch * nb, nn_ba,
                       (float*)nullptr);
    if (dev_err()) return MR_ERR_DEVICE;
    const int nblk = nblk_of(na) > 0 ? nblk_of(na) : 1;
    MutualPred pr{nn_ab, nn_ba, na, nb};
    hipLaunchKernelGGL(compact_count_kernel<MutualPred>, dim3(nblk, batch), dim3(256), 0, st, pr, na, blk, nblk);
    hipLaunchKernelGGL(compact_scatter_kernel<MutualPred>, dim3(nblk, batch), dim3(256), 0, st, pr, na,
                       (const int32_t*)blk, nblk, pairs, cap, n_pairs);
    return dev_err();
}

int mr_fast_reciprocal(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset, int32_t max_iters,
                       int32_t* pairs, int64_t cap, int64_t* n_pairs, int32_t* iter_active, void* ws,
                       size_t ws_bytes, void* stream) {
    int rc = validate_pair(a, b);
    if (rc) return rc;
    if (stride < 1 || offset < 0 || max_iters < 0) return MR_ERR_PARAM;
    if (!pairs || !n_pairs) return MR_ERR_NULL;
    const int64_t ns = seed_count(a->h, a->w, stride, offset);
    if (cap < ns) return MR_ERR_CAPACITY;
    const int64_t n1 = npix(a), n2 = npix(b);
    const FastLayout L = fast_layout(a->batch, ns, n1);
    if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int batch = a->batch;
    const int64_t slot = ns > 0 ? ns : 1;
    uint64_t* kf[2] = {at<uint64_t>(ws, L.keys_f[0]), at<uint64_t>(ws, L.keys_f[1])};
    uint64_t* kb[2] = {at<uint64_t>(ws, L.keys_b[0]), at<uint64_t>(ws, L.keys_b[1])};
    int32_t* fr[2] = {at<int32_t>(ws, L.front[0]), at<int32_t>(ws, L.front[1])};
    int32_t* cnt[2] = {at<int32_t>(ws, L.cnt[0]), at<int32_t>(ws, L.cnt[1])};
    int32_t* state = at<int32_t>(ws, L.state);
    int32_t* blk = at<int32_t>(ws, L.blk);

    InitArgs ia;
    ia.state = state; ia.n1 = n1; ia.w = a->w; ia.stride = stride; ia.offset = offset;
    ia.nx = (int32_t)(offset < a->w ? (a->w - 1 - offset) / stride + 1 : 0);
    ia.nseeds = (int32_t)ns;
    ia.front0 = fr[0]; ia.keys_f0 = kf[0]; ia.keys_b0 = kb[0]; ia.slot_stride = slot;
    ia.cnt0 = cnt[0]; ia.cnt1 = cnt[1];
    const int64_t init_n = n1 > ns ? n1 : ns;
    hipLaunchKernelGGL(fast_init_kernel, dim3(grid_1d(init_n > 0 ? init_n : 1), batch), dim3(256), 0, st, ia);
    if (dev_err()) return MR_ERR_DEVICE;

    if (n1 > 0 && n2 > 0 && ns > 0) {
        const int gx = nn_grid_x(ns, batch);
        const int cyc_grid = grid_1d(ns);
        for (int t = 0; t < max_iters; ++t) {
            const int c = t & 1, x = c ^ 1;
            NNArgs f = nn_args(a, b);
            f.qsrc = Q_LIST; f.qlist = fr[c]; f.qlist_stride = slot;
            f.dev_count = cnt[c]; f.count_stride = 1;
            f.keys = kf[c]; f.keys_stride = slot;
            if (iter_active) { f.active_out = iter_active + t; f.active_stride = max_iters; }
            f.zero_count = cnt[x]; f.zero_stride = 1;
            if ((rc = launch_nn(f, a->dtype, batch, gx, st))) return rc;
            NNArgs r = nn_args(b, a);
            r.qsrc = Q_KEYS; r.qlist = kf[c]; r.qlist_stride = slot;
            r.dev_count = cnt[c]; r.count_stride = 1;
            r.keys = kb[c]; r.keys_stride = slot;
            if ((rc = launch_nn(r, a->dtype, batch, gx, st))) return rc;
            CycleArgs ca;
            ca.front = fr[c]; ca.keys_f = kf[c]; ca.keys_b = kb[c];
            ca.keys_f_next = kf[x]; ca.keys_b_next = kb[x]; ca.front_next = fr[x];
            ca.cnt = cnt[c]; ca.cnt_next = cnt[x]; ca.state = state;
            ca.slot_stride = slot; ca.n1 = n1; ca.last = (t == max_iters - 1);
            hipLaunchKernelGGL(fast_cycle_kernel, dim3(cyc_grid, batch), dim3(256), 0, st, ca);
            if (dev_err()) return MR_ERR_DEVICE;
        }
    } else if (iter_active && max_iters > 0) {
        // nothing to search: every iteration has no live pixel
        const int64_t n = (int64_t)batch * max_iters;
        hipLaunchKernelGGL(fill_i32_kernel, dim3(grid_1d(n)), dim3(256), 0, st, iter_active, n, 0);
        if (dev_err()) return MR_ERR_DEVICE;
    }
    const int nblk = nblk_of(n1) > 0 ? nblk_of(n1) : 1;
    FastPred pr{state, n1};
    hipLaunchKernelGGL(compact_count_kernel<FastPred>, dim3(nblk, batch), dim3(256), 0, st, pr, n1, blk, nblk);
    hipLaunchKernelGGL(compact_scatter_kernel<FastPred>, dim3(nblk, batch), dim3(256), 0, st, pr, n1,
                       (const int32_t*)blk, nblk, pairs, cap, n_pairs);
    return dev_err();
}

int mr_profile_begin(int32_t max_launches) {
    if (g_prof.on || max_launches < 1) return MR_ERR_PARAM;
    g_prof.ev = static_cast<hipEvent_t*>(calloc((size_t)2 * max_launches, sizeof(hipEvent_t)));
    if (!g_prof.ev) return MR_ERR_DEVICE;
    for (int i = 0; i < 2 * max_launches; ++i) {
        if (hipEventCreate(&g_prof.ev[i]) != hipSuccess) {
            for (int k = 0; k < i; ++k) (void)hipEventDestroy(g_prof.ev[k]);
            free(g_prof.ev);
            g_prof.ev = nullptr;
            return MR_ERR_DEVICE;
        }
    }
    g_prof.cap = max_launches;
    g_prof.used = 0;
    g_prof.on = true;
    return MR_OK;
}

int mr_profile_end(double* total_ms, int64_t* launches) {
    if (!g_prof.on) return MR_ERR_PARAM;
    double tot = 0.0;
    int rc = MR_OK;
    for (int i = 0; i < g_prof.used; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess)
            rc = MR_ERR_DEVICE;
        tot += ms;
    }
    for (int i = 0; i < 2 * g_prof.cap; ++i) (void)hipEventDestroy(g_prof.ev[i]);
    free(g_prof.ev);
    if (total_ms) *total_ms = tot;
    if (launches) *launches = g_prof.used;
    g_prof = Profiler();
    return rc;
}

}  // extern "C"

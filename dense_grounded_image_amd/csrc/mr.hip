// mr.hip -- dense NN search and reciprocal matching for MI355X (gfx950, CDNA4).
//
// One similarity/argmax kernel serves every descriptor entry point (pointmaps have
// their own VALU kernel, point_nn_kernel, further down): a block of queries
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
//  - The matching loss the descriptors are trained with, InfoNCE over
//    ground-truth pairs ("MASt3R dissection", section 3), and its gradient: the
//    same similarity tiles with a log-sum-exp epilogue (lse_partial_kernel), and
//    softmax-weighted sums formed on the matrix cores (nce_grad_kernel).
//
// Layout of the MFMA operands (wave64, 32x32 output tile):
//  - lane l holds output column j = l & 31 (a query) and the 16 rows
//    i = 8*(v >> 2) + 4*(l >> 5) + (v & 3), v = 0..15 (database rows), so the
//    rows a lane sees rise with v and with the tile index;
//  - fp32 maps use V_MFMA_F32_32X32X2_F32 in P = ceil(d/2) steps; in step s
//    lane half h = l >> 5 supplies component c = P*h + s of its row;
//  - bf16 maps use V_MFMA_F32_32X32X16_BF16 in P = ceil(d/16) steps; in step s
//    lane half h supplies components 8*(P*h + s) .. +7 (zero past d).
// A and B use the same component-to-k assignment, products commute, and the
// accumulation order depends only on k, so s(i, j) is bitwise identical
// whichever map is the query side.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <type_traits>

#include "mr.h"

// Scratch memory of mr_fast_reciprocal_static: a fixed array in device memory, one
// copy per GPU, held until the process ends.  Host code never passes this name to a
// kernel or a copy (on the host it is only a stand-in for the symbol): the device
// address comes from hipGetSymbolAddress, per device.
constexpr size_t kStaticScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxSegGroups = 512;   // database segments per query block (bounds atomic contention)
constexpr int kCompactChunk = 2048;  // elements per block in the ordered compaction
constexpr int kMaxD = 64;

// ---------------------------------------------------------------------------- launch log

// MR_LOG set to anything but "" or "0" in the environment (read once per process)
// makes every entry point print, on stderr, a line with its maps and parameters, one
// line per kernel launch (kernel, template arguments, grid, block, LDS bytes, stream)
// and a line with the status it returns.  Off, it costs one branch per launch.
bool log_on() {
    static const bool on = [] {
        const char* e = getenv("MR_LOG");
        return e && e[0] && strcmp(e, "0") != 0;
    }();
    return on;
}

// `where` is the launching function's __PRETTY_FUNCTION__: its trailing "[...]", when
// it is a template, gives the launcher's template arguments (which select the kernel's).
void log_launch(const char* kernel, const char* where, dim3 g, dim3 b, size_t lds, hipStream_t st) {
    const char* targs = strrchr(where, '[');
    fprintf(stderr, "[mr]   launch %s%s%s%s grid (%u,%u,%u) block (%u,%u,%u) lds %zu stream %p\n", kernel,
            targs ? " (launcher " : "", targs ? targs : "", targs ? ")" : "", g.x, g.y, g.z, b.x, b.y, b.z, lds,
            static_cast<void*>(st));
}

// Every kernel launch of the library goes through this macro.
#define MR_LAUNCH(K, GRID, BLOCK, LDS, ST, ...)                                       \
    do {                                                                              \
        const dim3 mr_grid_ = (GRID), mr_block_ = (BLOCK);                            \
        if (log_on()) log_launch(#K, __PRETTY_FUNCTION__, mr_grid_, mr_block_, (LDS), (ST)); \
        hipLaunchKernelGGL(K, mr_grid_, mr_block_, LDS, ST, __VA_ARGS__);             \
    } while (0)

const char* dtype_name(int dt) { return dt == MR_F32 ? "f32" : dt == MR_BF16 ? "bf16" : "?"; }

// One entry-point call in the log: its maps and parameters on entry, its status on return.
class CallLog {
public:
    __attribute__((format(printf, 5, 6))) CallLog(const char* name, const mr_map* a, const mr_map* b,
                                                  const char* fmt, ...)
        : name_(name) {
        if (!log_on()) return;
        char pa[96], pb[96], extra[160];
        va_list ap;
        va_start(ap, fmt);
        vsnprintf(extra, sizeof(extra), fmt, ap);
        va_end(ap);
        fprintf(stderr, "[mr] %s a %s b %s %s\n", name, map_str(a, pa, sizeof(pa)), map_str(b, pb, sizeof(pb)),
                extra);
    }
    int done(int status) const {
        if (log_on()) fprintf(stderr, "[mr] %s -> %d (%s)\n", name_, status, mr_status_str(status));
        return status;
    }

private:
    static const char* map_str(const mr_map* m, char* buf, size_t n) {
        if (!m) return "NULL";
        snprintf(buf, n, "%dx%dx%dx%d %s @%p", m->batch, m->h, m->w, m->d, dtype_name(m->dtype), m->data);
        return buf;
    }
    const char* name_;
};

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

__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
    const uint32_t lo = __shfl((uint32_t)x, src);
    const uint32_t hi = __shfl((uint32_t)(x >> 32), src);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
    uint32_t lo = __shfl_xor((uint32_t)x, m);
    uint32_t hi = __shfl_xor((uint32_t)(x >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------------------- operands

// How a similarity is computed on the matrix cores.
//  AR_F32 : fp32 maps, fp32 products, V_MFMA_F32_32X32X2_F32 (any d).
//  AR_BF16: bf16 maps, exact bf16 products, V_MFMA_F32_32X32X16_BF16.
//  AR_X3  : fp32 maps split exactly into three bf16 parts x = h + m + l (the
//           workgroup writes each staged row's planes [h m l][d] to LDS); the six products
//           hh, hm, mh, mm, hl, lh are summed on V_MFMA_F32_32X32X16_BF16.  The three
//           dropped products are below 2^-23 |x||y|, so the result matches an fp32
//           dot product to within its own rounding, at 2.7x the matrix-core rate.
//           Each map keeps one fixed product order (image 1: h h m h l m, image 2:
//           h m h l h m over the six product slots), so a pair's products meet at
//           the same k whichever map is the query: scores stay bitwise symmetric.
enum Arith { AR_F32 = 0, AR_BF16 = 1, AR_X3 = 2 };

template <int AR, int P> struct Operand;

template <int P> struct Operand<AR_F32, P> {
    float x[P];
    __device__ __forceinline__ void load(const void* base, int64_t row, bool valid, int h, int d, int) {
        const float* p = static_cast<const float*>(base) + row * d;
        if constexpr (P % 4 == 0) {
            // d == 2P: the lane's P components are contiguous and 16-byte aligned
            if (d == 2 * P) {
                const float4* p4 = reinterpret_cast<const float4*>(p + (valid ? P * h : 0));
#pragma unroll
                for (int i = 0; i < P / 4; ++i) {
                    const float4 v = p4[i];
                    x[4 * i] = valid ? v.x : 0.0f;
                    x[4 * i + 1] = valid ? v.y : 0.0f;
                    x[4 * i + 2] = valid ? v.z : 0.0f;
                    x[4 * i + 3] = valid ? v.w : 0.0f;
                }
                return;
            }
        }
        // generic d: out-of-range components read the row's first element, then select 0
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int c = P * h + s;
            const bool ok = valid && c < d;
            const float t = p[ok ? c : 0];
            x[s] = ok ? t : 0.0f;
        }
    }
    __device__ __forceinline__ f32x16 mfma(const Operand& b, f32x16 acc) const {
#pragma unroll
        for (int s = 0; s < P; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(x[s], b.x[s], acc, 0, 0, 0);
        return acc;
    }
};

template <int P> struct Operand<AR_BF16, P> {
    bf16x8 x[P];
    __device__ __forceinline__ void load(const void* base, int64_t row, bool valid, int h, int d, int) {
        const uint16_t* p = static_cast<const uint16_t*>(base) + row * d;
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int c = 8 * (P * h + s);
            const bool ok = valid && c < d;
            u32x4 raw = *reinterpret_cast<const u32x4*>(p + (ok ? c : 0));
            if (!ok) raw = u32x4{0u, 0u, 0u, 0u};
            x[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    // Database side only: k-slots past d take the row's first chunk instead of zeros.
    // The query operand is zero in those slots and the maps are finite, so the
    // products there are +-0 and every score is unchanged (up to the sign of an
    // exact zero, which compares equal).  `tile` is the tile's first row (uniform);
    // off[s] the lane's byte offset in the tile (db_offsets).
    __device__ __forceinline__ void load_db(const char* tile, const int (&off)[P]) {
#pragma unroll
        for (int s = 0; s < P; ++s) x[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + off[s]));
    }
    static __device__ __forceinline__ void db_offsets(int jl, int h, int d, int (&off)[P]) {
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int c = 8 * (P * h + s);
            off[s] = (jl * d + (c < d ? c : 0)) * 2;
        }
    }
    __device__ __forceinline__ f32x16 mfma(const Operand& b, f32x16 acc) const {
#pragma unroll
        for (int s = 0; s < P; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[s], b.x[s], acc, 0, 0, 0);
        return acc;
    }
};

// Plane (0 = h, 1 = m, 2 = l) feeding product slot p for a map of the given role.
__host__ __device__ __forceinline__ constexpr int x3_plane(int role, int p) {
    return role == 1 ? (p == 2 || p == 5 ? 1 : (p == 4 ? 2 : 0))
                     : (p == 1 || p == 5 ? 1 : (p == 3 ? 2 : 0));
}

// Exact split of fp32 values into three bf16 parts v = h + m + l (round to nearest
// even at each step; each difference is exact in fp32), for four values at once: each
// plane comes out as two words of two bf16 (value 2i in the low half).  A conversion
// rounds a pair of values, each exactly as a scalar conversion would.
__device__ __forceinline__ void split3x4(float v0, float v1, float v2, float v3, uint2 (&pl)[3]) {
    f32x2 a = {v0, v1}, b = {v2, v3};
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const bf16x2 ha = __builtin_convertvector(a, bf16x2);
        const bf16x2 hb = __builtin_convertvector(b, bf16x2);
        pl[k] = uint2{__builtin_bit_cast(uint32_t, ha), __builtin_bit_cast(uint32_t, hb)};
        a = a - __builtin_convertvector(ha, f32x2);
        b = b - __builtin_convertvector(hb, f32x2);
    }
}

// P = 6d/16 steps (d = 8P/3); slot q = 16*s + 8*h + e holds product type q / d and
// component q % d.  A staged database tile holds each row as planes [h | m | l] of d
// bf16 (written by the workgroup from the fp32 map); query rows are split in
// registers.  The offsets are compile-time for each lane half.
template <int P> struct Operand<AR_X3, P> {
    static constexpr int D = 8 * P / 3;
    bf16x8 x[P];
    static __device__ __forceinline__ constexpr int offset(int role, int s, int h) {
        return x3_plane(role, (16 * s + 8 * h) / D) * D + (16 * s + 8 * h) % D;
    }
    // from a staged tile: planes [row][3][D]
    __device__ __forceinline__ void load(const void* base, int64_t row, bool valid, int h, int, int role) {
        const uint16_t* p = static_cast<const uint16_t*>(base) + row * 3 * D;
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int o0 = role == 1 ? offset(1, s, 0) : offset(2, s, 0);
            const int o1 = role == 1 ? offset(1, s, 1) : offset(2, s, 1);
            const int off = h ? o1 : o0;
            u32x4 raw = *reinterpret_cast<const u32x4*>(p + (valid ? off : 0));
            if (!valid) raw = u32x4{0u, 0u, 0u, 0u};
            x[s] = __builtin_bit_cast(bf16x8, raw);
        }
    }
    // from an fp32 row of the map, split here (fetch_f32 + split_f32, which callers may
    // separate to keep the row's loads in flight meanwhile)
    __device__ __forceinline__ void load_f32(const float* rowp, bool valid, int h, int role) {
        float4 raw[D / 4];
        fetch_f32(rowp, valid, raw);
        split_f32(raw, h, role);
    }
    static __device__ __forceinline__ void fetch_f32(const float* rowp, bool valid, float4 (&raw)[D / 4]) {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) raw[i] = valid ? reinterpret_cast<const float4*>(rowp)[i] : float4{0.f, 0.f, 0.f, 0.f};
    }
    __device__ __forceinline__ void split_f32(const float4 (&raw)[D / 4], int h, int role) {
        uint32_t pl[3][D / 2];   // planes, two bf16 per word
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            const float4 v = raw[i];
            uint2 a[3];
            split3x4(v.x, v.y, v.z, v.w, a);
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                pl[k][2 * i] = a[k].x;
                pl[k][2 * i + 1] = a[k].y;
            }
        }
#pragma unroll
        for (int s = 0; s < P; ++s) {
            const int o0 = role == 1 ? offset(1, s, 0) : offset(2, s, 0);
            const int o1 = role == 1 ? offset(1, s, 1) : offset(2, s, 1);
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t w0 = pl[o0 / D][(o0 % D) / 2 + e];
                const uint32_t w1 = pl[o1 / D][(o1 % D) / 2 + e];
                w[e] = h ? w1 : w0;
            }
            x[s] = __builtin_bit_cast(bf16x8, w);
        }
    }
    __device__ __forceinline__ f32x16 mfma(const Operand& b, f32x16 acc) const {
#pragma unroll
        for (int s = 0; s < P; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[s], b.x[s], acc, 0, 0, 0);
        return acc;
    }
    // step s alone (the same instruction and order as mfma, for interleaving chains)
    __device__ __forceinline__ f32x16 step(int s, const Operand& b, f32x16 acc) const {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(x[s], b.x[s], acc, 0, 0, 0);
    }
};

template <int AR> struct ArithTraits;
// tile_best: the streaming pass keeps each lane's best score and the tile it lies in
// (a short epilogue, for arithmetics whose matrix-core step is short next to it); a
// second kernel recomputes that tile to find the row.  Otherwise the pass keeps the
// row itself with a keyed maximum.
template <> struct ArithTraits<AR_F32> {
    using elem = float; static constexpr int row_mult = 1; static constexpr int qt = 4;
    static constexpr bool tile_best = false;
};
template <> struct ArithTraits<AR_BF16> {
    using elem = uint16_t; static constexpr int row_mult = 1; static constexpr int qt = 4;
    static constexpr bool tile_best = true;
};
template <> struct ArithTraits<AR_X3> {
    using elem = float; static constexpr int row_mult = 1; static constexpr int qt = 3;
    static constexpr bool tile_best = false;
};

// Query tiles held per wave (fewer for long descriptors, to stay out of scratch).
template <int AR, int P> constexpr int qt_of() { return AR == AR_X3 && P > 9 ? 2 : ArithTraits<AR>::qt; }

// ---------------------------------------------------------------------------- NN kernel

enum QuerySource { Q_ALL = 0, Q_LIST = 1 };

struct NNArgs {
    const void* qmap;        // [batch][nq_rows][d]
    const void* dbmap;       // [batch][ndb][d]
    int64_t q_pair_elems;    // nq_rows * d
    int64_t db_pair_elems;   // ndb * d
    int32_t nq_rows;
    int32_t ndb;
    int32_t d;
    int32_t qsrc;            // QuerySource
    const int32_t* qlist;    // int32 rows (Q_LIST), [batch][qlist_stride]
    int64_t qlist_stride;
    const int32_t* dev_count;  // per-pair query count on the device, or NULL
    int64_t count_stride;
    int32_t host_count;        // query count when dev_count is NULL
    uint64_t* keys;            // [batch][keys_stride] results, merged with atomicMax
    int64_t keys_stride;
    int32_t q_role, db_role;   // 1 = image 1, 2 = image 2 (fixes the split product order)
    // pair graph: the query (database) map of pair b is map q_img[2b] (db_img[2b]) of
    // qmap (dbmap); NULL: map b
    const int32_t* q_img;
    const int32_t* db_img;
    // 0: grid (workgroups per pair, batch).  Otherwise a one-dimensional grid in which
    // all xcd_gx workgroups of a pair share one XCD (see xcd_packed_grid); batch is the
    // pair count.
    int32_t xcd_gx;
    int32_t batch;
};

// Map index of pair b in a stacked collection (a pair graph's edge table, or b itself).
__device__ __forceinline__ int64_t map_of(const int32_t* img, int pair) {
    return img ? (int64_t)img[2 * pair] : (int64_t)pair;
}

// Scores are compared after clearing their 4 lowest fp32 bits; that order, with
// the lowest row winning ties, is the NN rule of every kernel (both directions use
// it, so it is symmetric).  The cleared bits carry the row's place in the tile, so
// one integer max3 tree finds a tile's best candidate.
__device__ __forceinline__ float trunc4(float s) { return __int_as_float(__float_as_int(s) & ~15); }

// Row (within its 32-row tile) of accumulator register v in lane half h.
__device__ __forceinline__ int tile_row(int v, int h) { return 8 * (v >> 2) + 4 * h + (v & 3); }

// Best key of one tile for one lane: (score bits with 4 low bits cleared) | (15 - v).
// Valid whenever the lane's best score is >= 0 (float bits then order as ints).
template <bool RAGGED>
__device__ __forceinline__ int tile_key(const f32x16& acc, int t, int h, int ndb) {
    int k[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        k[v] = (__float_as_int(acc[v]) & ~15) | (15 - v);
        if (RAGGED && t * 32 + tile_row(v, h) >= ndb) k[v] = INT_MIN;
    }
    const int a0 = max(max(k[0], k[1]), k[2]), a1 = max(max(k[3], k[4]), k[5]);
    const int a2 = max(max(k[6], k[7]), k[8]), a3 = max(max(k[9], k[10]), k[11]);
    const int a4 = max(max(k[12], k[13]), k[14]);
    return max(max(max(a0, a1), a2), max(max(a3, a4), k[15]));
}

// The same rule, exactly, for lanes whose best score is negative (rare): a running
// maximum of trunc4(s) over rows in increasing order, strict '>'.
template <bool RAGGED>
__device__ __forceinline__ void tile_exact(const f32x16& acc, int t, int h, int ndb, float& bv, int& bt) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        const float s = trunc4(acc[v]);
        bool gt = s > bv;
        if (RAGGED) gt = gt && (t * 32 + tile_row(v, h) < ndb);
        bv = gt ? s : bv;
        bt = gt ? (t * 16 + v) : bt;
    }
}

// Tile-level form of the same rule: a running maximum of trunc4(tile maximum) over
// tiles in increasing order, strict '>', remembering the tile.  trunc4 is monotone,
// so trunc4 of the tile's maximum is the tile's best compared score, and the first
// tile reaching a lane's final best holds that lane's NN (the lowest such row is
// found later by recomputing that one tile).  IEEE maximum needs no operand
// canonicalisation and treats every finite input exactly; the running best is
// folded into the tree, so "improved" is a plain inequality.
template <bool RAGGED>
__device__ __forceinline__ void tile_track(const f32x16& acc, int t, int h, int ndb, float& bv, int& bt) {
    float k[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) k[v] = (RAGGED && t * 32 + tile_row(v, h) >= ndb) ? -INFINITY : acc[v];
    auto mx3 = [](float a, float b, float c) {
        return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
    };
    const float m0 = mx3(k[0], k[1], k[2]), m1 = mx3(k[3], k[4], k[5]), m2 = mx3(k[6], k[7], k[8]);
    const float m3 = mx3(k[9], k[10], k[11]), m4 = mx3(k[12], k[13], k[14]), m5 = mx3(k[15], bv, m0);
    const float m = trunc4(mx3(mx3(m1, m2, m3), m4, m5));
    bt = m != bv ? t : bt;
    bv = m;
}

// Per-lane running state of a streamed database segment: one entry per query tile
// j, updated once per 32-row database tile t (RAGGED: rows at or past ndb are
// masked).  step() takes the ragged flag at run time.
enum Epilogue { EP_KEY = 0, EP_EXACT = 1, EP_TILE = 2, EP_LSE = 3 };

// Keyed row maximum: (score, row) of the NN while the lane's best score is >= 0.
template <int QT> struct KeyBest {
    static constexpr int kind = EP_KEY;
    static constexpr int valu = 27;   // vector instructions per tile, for scheduling
    int bk[QT], bt[QT];
    __device__ __forceinline__ KeyBest() {
#pragma unroll
        for (int j = 0; j < QT; ++j) { bk[j] = INT_MIN; bt[j] = -1; }
    }
    __device__ __forceinline__ void keep(int km, int t, int j) {
        const bool gt = km > (bk[j] | 15);   // strictly better score: earliest tile wins ties
        bk[j] = gt ? km : bk[j];
        bt[j] = gt ? t : bt[j];
    }
    template <bool RAGGED>
    __device__ __forceinline__ void tile(const f32x16& acc, int t, int h, int ndb, int j) {
        keep(tile_key<RAGGED>(acc, t, h, ndb), t, j);
    }
    __device__ __forceinline__ void step(const f32x16& acc, int t, int h, int ndb, int j, bool ragged) {
        keep(ragged ? tile_key<true>(acc, t, h, ndb) : tile_key<false>(acc, t, h, ndb), t, j);
    }
};

// Exact row maximum (any sign); bx = 16 * tile + accumulator register.
template <int QT> struct ExactBest {
    static constexpr int kind = EP_EXACT;
    float bv[QT];
    int bx[QT];
    __device__ __forceinline__ ExactBest() {
#pragma unroll
        for (int j = 0; j < QT; ++j) { bv[j] = -INFINITY; bx[j] = -1; }
    }
    template <bool RAGGED>
    __device__ __forceinline__ void tile(const f32x16& acc, int t, int h, int ndb, int j) {
        tile_exact<RAGGED>(acc, t, h, ndb, bv[j], bx[j]);
    }
    __device__ __forceinline__ void step(const f32x16& acc, int t, int h, int ndb, int j, bool ragged) {
        if (ragged) tile<true>(acc, t, h, ndb, j);
        else tile<false>(acc, t, h, ndb, j);
    }
};

// Tile-level maximum: best compared score and the first tile reaching it.
template <int QT> struct TileBest {
    static constexpr int kind = EP_TILE;
    static constexpr int valu = 12;   // vector instructions per tile, for scheduling
    float bv[QT];
    int bt[QT];
    __device__ __forceinline__ TileBest() {
#pragma unroll
        for (int j = 0; j < QT; ++j) { bv[j] = -INFINITY; bt[j] = -1; }
    }
    template <bool RAGGED>
    __device__ __forceinline__ void tile(const f32x16& acc, int t, int h, int ndb, int j) {
        tile_track<RAGGED>(acc, t, h, ndb, bv[j], bt[j]);
    }
    __device__ __forceinline__ void step(const f32x16& acc, int t, int h, int ndb, int j, bool ragged) {
        if (ragged) tile<true>(acc, t, h, ndb, j);
        else tile<false>(acc, t, h, ndb, j);
    }
};

// Group-level maximum (the rows of the fused row + column pass): per lane and query
// tile, the raw maximum over the current group of b tiles (one max3 tree per tile,
// nothing else), and at the end of each group (close) the best compared score and the
// first group reaching it, named by the caller's group index.  trunc4 is monotone, so the
// group's compared maximum is trunc4 of its raw maximum, and the lane's NN is the
// lowest row of that group whose compared score equals the best (found later by
// recomputing the group).
template <int QT> struct GroupBest {
    float gm[QT], bv[QT];
    int bt[QT];
    __device__ __forceinline__ GroupBest() {
#pragma unroll
        for (int j = 0; j < QT; ++j) { gm[j] = -INFINITY; bv[j] = -INFINITY; bt[j] = -1; }
    }
    template <bool RAGGED>
    __device__ __forceinline__ void tile(const f32x16& acc, int t, int h, int ndb, int j) {
        float k[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) k[v] = (RAGGED && t * 32 + tile_row(v, h) >= ndb) ? -INFINITY : acc[v];
        auto mx3 = [](float a, float b, float c) {
            return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
        };
        const float m0 = mx3(k[0], k[1], k[2]), m1 = mx3(k[3], k[4], k[5]), m2 = mx3(k[6], k[7], k[8]);
        const float m3 = mx3(k[9], k[10], k[11]), m4 = mx3(k[12], k[13], k[14]), m5 = mx3(k[15], gm[j], m0);
        gm[j] = mx3(mx3(m1, m2, m3), m4, m5);
    }
    __device__ __forceinline__ void step(const f32x16& acc, int t, int h, int ndb, int j, bool ragged) {
        if (ragged) tile<true>(acc, t, h, ndb, j);
        else tile<false>(acc, t, h, ndb, j);
    }
    __device__ __forceinline__ void close(int tg) {
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            const float m = trunc4(__builtin_elementwise_maximum(gm[j], bv[j]));
            bt[j] = m != bv[j] ? tg : bt[j];
            bv[j] = m;
            gm[j] = -INFINITY;
        }
    }
};

// Online log-sum-exp of a query's scores over the database rows (the softmax
// normaliser of the matching loss), in base 2: with k2 = log2(e) / tau and
// z = score * k2, the state is an integer offset m and s = the sum over the rows seen
// of 2^(z - m), each exponent formed as fma(score, k2, -m) (one rounding).  m starts
// at -inf and is raised only when a tile's terms would sum past 2^64 (the first tile,
// or a rise of the scores by more than 64 / k2): it becomes the integer just above
// the tile's largest z, and s is rescaled by 2^(m_old - m_new), an exact power of
// two.  Between raises the terms may exceed 1 (by at most 2^64 per tile), so s needs
// no per-tile maximum, rescale or second exponential; a raise recomputes that tile's
// terms.  s is a compensated (Kahan) sum with compensation c, so its error stays at a
// few units of fp32 rounding however long the segment.
__device__ __forceinline__ float scale_pow2(float x, float e) {   // x * 2^e, e an integer
    return __builtin_ldexpf(x, (int)e);
}

template <int QT> struct LseSum {
    static constexpr int kind = EP_LSE;
    static constexpr int valu = 52;   // vector instructions per tile, for scheduling
    float m[QT], s[QT], c[QT];
    float k2;
    __device__ __forceinline__ explicit LseSum(float k2_) : k2(k2_) {
#pragma unroll
        for (int j = 0; j < QT; ++j) { m[j] = -INFINITY; s[j] = 0.0f; c[j] = 0.0f; }
    }
    template <bool RAGGED>
    __device__ __forceinline__ void tile(const f32x16& acc, int t, int h, int ndb, int j) {
        float k[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) k[v] = (RAGGED && t * 32 + tile_row(v, h) >= ndb) ? -INFINITY : acc[v];
        auto terms = [&](float off) {
            float e[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) e[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(k[v], k2, off));
#pragma unroll
            for (int w = 8; w >= 1; w >>= 1)
#pragma unroll
                for (int v = 0; v < w; ++v) e[v] += e[v + w];
            return e[0];
        };
        float S = terms(-m[j]);
        const bool raise = !(S <= 0x1p64f);   // m = -inf (inf or NaN terms), or the scores rose
        // rare: a wave-uniform branch, so the common tile runs none of it
        if (__builtin_amdgcn_ballot_w64(raise)) {
            auto mx3 = [](float a, float b, float c) {
                return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
            };
            const float m0 = mx3(k[0], k[1], k[2]), m1 = mx3(k[3], k[4], k[5]), m2 = mx3(k[6], k[7], k[8]);
            const float m3 = mx3(k[9], k[10], k[11]), m4 = mx3(k[12], k[13], k[14]);
            const float mt = mx3(mx3(m1, m2, m3), m4, __builtin_elementwise_maximum(k[15], m0));
            // the other lanes keep their offset; a lane with no row yet (ragged tiles
            // only) keeps m = -inf and adds nothing
            const float mn = raise ? __builtin_elementwise_maximum(m[j], __builtin_ceilf(mt * k2)) : m[j];
            if (mn != m[j]) {
                if (m[j] != -INFINITY) {
                    s[j] = scale_pow2(s[j], m[j] - mn);
                    c[j] = scale_pow2(c[j], m[j] - mn);
                }
                m[j] = mn;
            }
            const float S2 = terms(mn == -INFINITY ? 0.0f : -mn);
            S = raise ? S2 : S;
        }
        const float y = S - c[j];
        const float tot = s[j] + y;
        c[j] = (tot - s[j]) - y;
        s[j] = tot;
    }
    __device__ __forceinline__ void step(const f32x16& acc, int t, int h, int ndb, int j, bool ragged) {
        if (ragged) tile<true>(acc, t, h, ndb, j);
        else tile<false>(acc, t, h, ndb, j);
    }
};

template <int AR> __device__ __forceinline__ const void* pair_base(const void* p, int64_t elems, int64_t map) {
    return static_cast<const typename ArithTraits<AR>::elem*>(p) + map * elems * ArithTraits<AR>::row_mult;
}

// Bytes of one map row as the kernel reads it, and an upper bound for the template.
template <int AR> __device__ __forceinline__ int row_bytes(int d) {
    return (int)sizeof(typename ArithTraits<AR>::elem) * ArithTraits<AR>::row_mult * d;
}
template <int AR, int P> constexpr int max_row_bytes() {        // a map row in memory
    return AR == AR_F32 ? 8 * P : (AR == AR_BF16 ? 32 * P : 32 * P / 3);
}
template <int AR, int P> constexpr int lds_row_bytes() {        // a staged row (X3: three planes)
    return AR == AR_X3 ? 16 * P : max_row_bytes<AR, P>();
}

// Scheduling hint for a loop body of N matrix instructions: issue each one followed by
// V vector instructions.  A wave issues in order, and one that reaches a matrix
// instruction while the matrix core is busy stalls there; vector work placed between
// the matrix instructions of the same wave runs while they execute.
template <int N, int V>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, V, 0);   // then V VALU
    }
}

// One workgroup streams 32-row database tiles through a double-buffered LDS stage
// (one cooperative 16-byte-chunk copy per tile, one barrier per tile); each of its
// four waves multiplies the staged tile against its own QT query tiles held in
// registers; the per-lane state ep (one of the epilogue states above) takes each
// product tile.
constexpr int kSplitValu = 26;   // vector instructions of one lane's split-fp32 staging (a chunk of four)

template <int AR, int P, int QT, class Ep>
__device__ __forceinline__ void stream_tiles(const char* __restrict__ dbytes, int rb, int t0, int t1, int ndb,
                                             char* lds, const Operand<AR, P> (&q)[QT],
                                             int nact, int h, int jl, int d, int role, Ep& ep) {
    constexpr int MAXC = (32 * max_row_bytes<AR, P>() / 16 + kThreads - 1) / kThreads;
    constexpr int BUF = 32 * lds_row_bytes<AR, P>();
    const int tile_bytes = 32 * rb;
    const int nchunk = tile_bytes >> 4;
    const int nt = t1 - t0;
    u32x4 stage0[MAXC], stage1[MAXC];

    auto fetch = [&](int t, u32x4 (&stage)[MAXC]) {
        const int64_t tb = (int64_t)t * tile_bytes;
        const int64_t limit = (int64_t)ndb * rb;   // bytes of real rows
        if constexpr (AR == AR_X3) {
            // rows are whole 16-byte chunks: every lane loads one chunk per slot, lanes
            // past the tile's real rows (or past the tile) a copy of its last real chunk,
            // so the load count never depends on the lane or the tile and the compiler
            // waits only for the older stage.  Rows of a ragged tile past the map's end
            // then hold finite stale data, which the ragged epilogue masks.
            const int rows = ndb - t * 32 < 32 ? ndb - t * 32 : 32;
            const int nvalid = rows * (rb >> 4);
            const char* base = dbytes + tb;
#pragma unroll
            for (int c = 0; c < MAXC; ++c) {
                const int ch = threadIdx.x + c * kThreads;
                stage[c] = *reinterpret_cast<const u32x4*>(base + (ch < nvalid ? ch : nvalid - 1) * 16);
            }
            return;
        }
        if ((t + 1) * 32 <= ndb) {
            // a whole tile: every chunk is in bounds (wave-uniform base, per-lane offset)
            const char* base = dbytes + tb;
#pragma unroll
            for (int c = 0; c < MAXC; ++c) {
                const int ch = threadIdx.x + c * kThreads;
                if (ch < nchunk) stage[c] = *reinterpret_cast<const u32x4*>(base + ch * 16);
            }
            return;
        }
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = threadIdx.x + c * kThreads;
            const int64_t off = tb + (int64_t)ch * 16;
            u32x4 v = {0u, 0u, 0u, 0u};
            if (ch < nchunk && off + 16 <= limit) {
                v = *reinterpret_cast<const u32x4*>(dbytes + off);
            } else if (ch < nchunk && off < limit) {
                // the chunk holding the end of the last row (row sizes are multiples of 4 bytes)
                const uint32_t* w = reinterpret_cast<const uint32_t*>(dbytes + off);
                const int nw = (int)((limit - off) >> 2);
                v.x = w[0];
                if (nw > 1) v.y = w[1];
                if (nw > 2) v.z = w[2];
            }
            stage[c] = v;
        }
    };
    // split fp32 staging in three parts, one per query tile's chain (part k forms plane
    // k; the last part also writes the three planes to LDS)
    struct Split { f32x2 a, b; uint2 pl[3]; };
    auto put_part = [&](int k, int buf, const u32x4 (&stage)[MAXC], Split& sp) {
        static_assert(AR != AR_X3 || MAXC == 1, "one chunk per lane");
        if (k == 0) {
            sp.a = f32x2{__uint_as_float(stage[0][0]), __uint_as_float(stage[0][1])};
            sp.b = f32x2{__uint_as_float(stage[0][2]), __uint_as_float(stage[0][3])};
        }
        const bf16x2 ha = __builtin_convertvector(sp.a, bf16x2);
        const bf16x2 hb = __builtin_convertvector(sp.b, bf16x2);
        sp.pl[k] = uint2{__builtin_bit_cast(uint32_t, ha), __builtin_bit_cast(uint32_t, hb)};
        if (k < 2) {
            sp.a = sp.a - __builtin_convertvector(ha, f32x2);
            sp.b = sp.b - __builtin_convertvector(hb, f32x2);
            return;
        }
        constexpr int D = 8 * P / 3;
        const int ch = threadIdx.x;
        const int cw = ch < nchunk ? ch : nchunk - 1;
        const int r = cw / (D / 4), c0 = (cw - r * (D / 4)) * 4;
        char* dst = lds + buf * BUF + r * 6 * D + c0 * 2;
#pragma unroll
        for (int q3 = 0; q3 < 3; ++q3) *reinterpret_cast<uint2*>(dst + q3 * 2 * D) = sp.pl[q3];
    };
    auto put = [&](int buf, const u32x4 (&stage)[MAXC]) {
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = threadIdx.x + c * kThreads;
            if constexpr (AR == AR_X3) {
                // four fp32 components -> their h, m, l bf16 in the row's three planes.
                // Branch-free: lanes past the tile's chunks hold the same chunk as the
                // tile's last lane (the fetch clamps both to the last real chunk) and write
                // it to the same place, so the staging can sit between matrix instructions.
                constexpr int D = 8 * P / 3;
                const int cw = ch < nchunk ? ch : nchunk - 1;
                const int r = cw / (D / 4), c0 = (cw - r * (D / 4)) * 4;
                uint2 a[3];
                split3x4(__uint_as_float(stage[c][0]), __uint_as_float(stage[c][1]),
                         __uint_as_float(stage[c][2]), __uint_as_float(stage[c][3]), a);
                char* dst = lds + buf * BUF + r * 6 * D + c0 * 2;
#pragma unroll
                for (int k = 0; k < 3; ++k) *reinterpret_cast<uint2*>(dst + k * 2 * D) = a[k];
            } else if (ch < nchunk) {
                *reinterpret_cast<u32x4*>(lds + buf * BUF + ch * 16) = stage[c];
            }
        }
    };

    // Full tiles of the split contraction with keyed epilogues run one (tile, query
    // tile) unit behind: the products of unit n are issued with the epilogue of unit
    // n - 1 between them, so the vector work runs while the matrix core is busy.  The
    // pending unit is (lag, lag_t, query tile QT - 1) across tiles.  Applying a unit to
    // a keyed state twice changes nothing (the comparison is strict, against the key
    // with its low bits set), so the first full tile's stand-in (all scores -inf,
    // whose keys are negative and never beat a lane's best once it is >= 0; a lane
    // whose best stays negative is recomputed exactly) needs no special case either.
    f32x16 lag;
#pragma unroll
    for (int v = 0; v < 16; ++v) lag[v] = -INFINITY;
    int lag_t = t0;
    bool pending = false;
    auto flush = [&]() {
        if (pending) ep.template tile<false>(lag, lag_t, h, ndb, QT - 1);
        pending = false;
    };

    // mid(k), k = 0, 1, 2: the parts of the next tile's staging (split fp32: the split
    // and its LDS write), issued inside compute -- on the interleaved path one part per
    // query tile's chain, between its matrix instructions, so that the vector work runs
    // while the matrix core is busy (the matrix core hides only a few vector
    // instructions behind each of its own, and none of another wave's)
    auto compute = [&](int i, auto&& mid) {
        const int t = t0 + i;
        const bool ragged = (t + 1) * 32 > ndb;
        Operand<AR, P> r;
        r.load(lds + (i & 1) * BUF, jl, true, h, d, role);
        if constexpr (AR == AR_X3 && Ep::kind == EP_KEY) {
            if (nact == QT && !ragged) {
                // the last query tile's chain accumulates straight into the pending
                // unit (whose previous value the first epilogue has consumed)
                f32x16 acc[QT > 1 ? QT - 1 : 1];
                constexpr int JM = QT > 1 ? 1 : 0;   // the chain that carries the staging
#pragma unroll
                for (int j = 0; j < QT; ++j) {
                    f32x16 x = {};
#pragma unroll
                    for (int st = 0; st < P; ++st) x = r.step(st, q[j], x);
                    if (j > 0) ep.template tile<false>(acc[j - 1], t, h, ndb, j - 1);
                    else ep.template tile<false>(lag, lag_t, h, ndb, QT - 1);
                    if (j < QT - 1) acc[j] = x;
                    else lag = x;
                    if constexpr (QT == 3) {
                        mid(j);
                        interleave_mfma_valu<P, (Ep::valu + kSplitValu / 3 + P - 1) / P>();
                    } else if (j == JM) {
                        mid(0); mid(1); mid(2);
                        interleave_mfma_valu<P, (Ep::valu + kSplitValu + P - 1) / P>();
                    } else {
                        interleave_mfma_valu<P, (Ep::valu + P - 1) / P>();
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
                lag_t = t;
                pending = true;
                return;
            }
            flush();
        }
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            if (j < nact) {
                f32x16 acc = {};
                acc = r.mfma(q[j], acc);
                ep.step(acc, t, h, ndb, j, ragged);
            }
        }
        mid(0); mid(1); mid(2);
    };

    if (nt <= 0) return;
    // tile i is fetched into registers two iterations before it is needed, written to
    // LDS buffer i&1 at the end of iteration i-1, and read after that iteration's barrier
    fetch(t0, stage0);
    put(0, stage0);
    if (AR == AR_X3) fetch(t0 + (nt > 1 ? 1 : 0), stage1);
    else if (nt > 1) fetch(t0 + 1, stage1);
    __syncthreads();
    // (split fp32: the fetches past the last tile re-read it, so that every iteration
    // issues the same loads)
    if constexpr (AR == AR_X3) {
        // the LDS write of the next tile runs inside the products of this one; past the
        // last tile it writes the re-read copy into the buffer nobody reads again
        Split sp;
        for (int i = 0; i < nt; i += 2) {
            fetch(t0 + (i + 2 < nt ? i + 2 : nt - 1), stage0);
            compute(i, [&](int k) { put_part(k, 1, stage1, sp); });
            __syncthreads();
            if (i + 1 >= nt) break;
            fetch(t0 + (i + 3 < nt ? i + 3 : nt - 1), stage1);
            compute(i + 1, [&](int k) { put_part(k, 0, stage0, sp); });
            __syncthreads();
        }
    } else {
        for (int i = 0; i < nt; i += 2) {
            if (i + 2 < nt) fetch(t0 + i + 2, stage0);
            compute(i, [](int) {});
            if (i + 1 < nt) put(1, stage1);
            __syncthreads();
            if (i + 1 >= nt) break;
            if (i + 3 < nt) fetch(t0 + i + 3, stage1);
            compute(i + 1, [](int) {});
            if (i + 2 < nt) put(0, stage0);
            __syncthreads();
        }
    }
    if constexpr (AR == AR_X3 && Ep::kind == EP_KEY) flush();
}

// One workgroup streams its database segment (bf16 rows) through a ring of three LDS
// stages of S tiles: global loads are issued two stages ahead of their LDS write,
// one barrier per stage.  Each wave multiplies the staged tiles against its own
// nact query tiles held in registers and hands each product tile to the per-lane
// state ep.  Loads and LDS writes are issued unconditionally -- stage indices past the
// end clamp to the last stage, chunks past the map's last row to that row's last
// chunk -- so that the compiler counts outstanding loads exactly and waits only for
// the oldest stage.  LDS rows past the map's end hold stale (finite) data; the
// ragged epilogue masks them.
constexpr int kStageTiles = 2;

template <int AR, int P, int S, int QT, class Ep>
__device__ __forceinline__ void stream_staged(const char* __restrict__ dbytes, int rb, int t0, int t1, int ndb,
                                              char* lds, const Operand<AR, P> (&q)[QT], int nact,
                                              int h, int jl, int d, int role, Ep& ep) {
    static_assert(AR == AR_BF16, "the staged ring holds bf16 rows");

    constexpr int NB = 3;
    constexpr int STAGE = S * 32 * lds_row_bytes<AR, P>();
    constexpr int MAXC = (S * 32 * max_row_bytes<AR, P>() / 16 + kThreads - 1) / kThreads;
    const int row_chunks = rb >> 4;
    const int nst = (t1 - t0 + S - 1) / S;
    u32x4 slot0[MAXC], slot1[MAXC];
    Operand<AR, P> opr[S];
    int off[P];
    Operand<AR, P>::db_offsets(jl, h, d, off);

    // chunks of stage k that hold real rows
    auto stage_chunks = [&](int k) {
        const int r0 = (t0 + S * k) * 32;
        const int nr = ndb - r0 < S * 32 ? ndb - r0 : S * 32;
        return nr * row_chunks;
    };
    auto fetch = [&](int k, u32x4 (&st)[MAXC]) {
        k = k < nst ? k : nst - 1;
        const int nch = stage_chunks(k);
        const char* src = dbytes + (int64_t)(t0 + S * k) * 32 * rb;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = threadIdx.x + c * kThreads;
            st[c] = *reinterpret_cast<const u32x4*>(src + (ch < nch ? ch : nch - 1) * 16);
        }
    };
    auto put = [&](int k, const u32x4 (&st)[MAXC]) {
        const int nch = stage_chunks(k < nst ? k : nst - 1);
        char* buf = lds + (k % NB) * STAGE;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int ch = threadIdx.x + c * kThreads;
            if (ch < nch) *reinterpret_cast<u32x4*>(buf + ch * 16) = st[c];
        }
    };
    // the S tiles of stage k, read into the A operands
    auto read = [&](int k) {
        const char* buf = lds + (k % NB) * STAGE;
#pragma unroll
        for (int x = 0; x < S; ++x) opr[x].load_db(buf + x * 32 * rb, off);
    };
    auto epilogue = [&](const f32x16& acc, int t, bool ragged, int j) { ep.step(acc, t, h, ndb, j, ragged); };
    auto compute = [&](int k) {
#pragma unroll
        for (int x = 0; x < S; ++x) {
            const int t = t0 + S * k + x;
            if (S == 1 || t < t1) {
                const bool ragged = (t + 1) * 32 > ndb;
                // one query tile at a time: the epilogue of tile j overlaps the
                // products of tile j+1
                if (nact == QT) {
#pragma unroll
                    for (int j = 0; j < QT; ++j) epilogue(opr[x].mfma(q[j], f32x16{}), t, ragged, j);
                } else {
#pragma unroll
                    for (int j = 0; j < QT; ++j)
                        if (j < nact) epilogue(opr[x].mfma(q[j], f32x16{}), t, ragged, j);
                }
            }
        }
    };

    if (nst <= 0) return;
    // stage k: global -> slot k&1 at iteration k-3 (the prologue for k < 3), LDS
    // buffer k%3 at iteration k-2, read and multiplied at iteration k
    fetch(0, slot0);
    fetch(1, slot1);
    put(0, slot0);
    fetch(2, slot0);
    put(1, slot1);
    __syncthreads();
    for (int k = 0; k < nst; k += 2) {
        // buffers of stages past the end are free: writing them is harmless
        fetch(k + 3, slot1);
        read(k);
        compute(k);
        put(k + 2, slot0);
        __syncthreads();
        if (k + 1 >= nst) break;
        fetch(k + 4, slot0);
        read(k + 1);
        compute(k + 1);
        put(k + 3, slot1);
        __syncthreads();
    }
}

// The workgroup-staged stream for an arithmetic: the LDS ring for bf16 rows; the
// plain double buffer for fp32 rows (measured faster for the long split contraction,
// whose nine matrix-core steps per tile already cover the staging latency).
template <int AR, int P, int QT, class Ep>
__device__ __forceinline__ void stream_db(const char* __restrict__ dbytes, int rb, int t0, int t1, int ndb, char* lds,
                                          const Operand<AR, P> (&q)[QT], int nact, int h, int jl, int d,
                                          int role, Ep& ep) {
    if constexpr (AR != AR_BF16)
        stream_tiles<AR, P>(dbytes, rb, t0, t1, ndb, lds, q, nact, h, jl, d, role, ep);
    else
        stream_staged<AR, P, kStageTiles>(dbytes, rb, t0, t1, ndb, lds, q, nact, h, jl, d, role, ep);
}

// Full work items of bf16 maps, without LDS or barriers: each wave reads the
// database operand straight from global memory (the four waves of a workgroup read
// the same tiles, so L1 serves all but the first) into a ring of D tiles issued D
// tiles ahead of their use.
template <int AR, int P, int D, int QT, class Ep>
__device__ __forceinline__ void stream_regs(const void* dbase, int t0, int t1,
                                            const Operand<AR, P> (&q)[QT], int h, int jl, int d,
                                            Ep& ep) {
    static_assert(AR == AR_BF16, "direct database operands are bf16 only");
    Operand<AR, P> r[D];
    int off[P];
    Operand<AR, P>::db_offsets(jl, h, d, off);
    const char* dbytes = static_cast<const char*>(dbase);
    const int64_t tile_bytes = (int64_t)64 * d;   // 32 rows of 2d bytes
    const int tlast = t1 - 1;
#pragma unroll
    for (int u = 0; u < D; ++u) {
        const int tt = t0 + u < tlast ? t0 + u : tlast;
        r[u].load_db(dbytes + tt * tile_bytes, off);
    }
    auto compute = [&](const Operand<AR, P>& rr, int tt) {
        f32x16 acc[QT];
#pragma unroll
        for (int j = 0; j < QT; ++j) acc[j] = rr.mfma(q[j], f32x16{});
#pragma unroll
        for (int j = 0; j < QT; ++j) ep.template tile<false>(acc[j], tt, h, 0, j);
    };
    // whole groups of D tiles: no branch inside, refills clamped, so the compiler
    // counts outstanding loads exactly
    // Inside a group the epilogue runs one (tile, query tile) unit behind the matrix
    // products: the products of unit n are issued, then the epilogue of unit n - 1,
    // whose results are complete by then, fills the matrix core's busy cycles.
    int t = t0;
    for (; t + D <= t1; t += D) {
        f32x16 prev;
#pragma unroll
        for (int u = 0; u < D; ++u) {
#pragma unroll
            for (int j = 0; j < QT; ++j) {
                const f32x16 acc = r[u].mfma(q[j], f32x16{});
                if (j > 0) ep.template tile<false>(prev, t + u, h, 0, j - 1);
                else if (u > 0) ep.template tile<false>(prev, t + u - 1, h, 0, QT - 1);
                prev = acc;
                interleave_mfma_valu<P, (Ep::valu + P - 1) / P>();
                __builtin_amdgcn_sched_barrier(0);
            }
            const int tn = t + u + D < tlast ? t + u + D : tlast;
            r[u].load_db(dbytes + tn * tile_bytes, off);
        }
        ep.template tile<false>(prev, t + D - 1, h, 0, QT - 1);
    }
    // the last t1 - t < D tiles are already in the ring
#pragma unroll
    for (int u = 0; u < D - 1; ++u)
        if (t + u < t1) compute(r[u], t + u);
}

// Small frontiers (all live queries fit in one wave): every wave of the workgroup
// holds the same queries and streams its own database segment straight from global
// memory, one tile ahead in registers, with no LDS staging and no barriers.
// Split fp32 rows are fetched a tile ahead and split after the current tile's
// products, so each tile's load is in flight during the previous tile's products.
template <int AR, int P, int QT, class Ep>
__device__ __forceinline__ void stream_direct(const void* dbase, int t0, int t1, int ndb,
                                              const Operand<AR, P> (&q)[QT],
                                              int nact, int h, int jl, int d, int role, Ep& ep) {
    if (t0 >= t1) return;
    auto row_of = [&](int t) { return (int64_t)t * 32 + jl; };
    auto compute = [&](const Operand<AR, P>& r, int t) {
        const bool ragged = (t + 1) * 32 > ndb;
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            if (j < nact) {
                f32x16 acc = {};
                acc = r.mfma(q[j], acc);
                ep.step(acc, t, h, ndb, j, ragged);
            }
        }
    };
    if constexpr (AR == AR_X3) {
        constexpr int D = Operand<AR, P>::D;
        float4 raw[D / 4];
        auto fetch = [&](int t) {
            const int64_t row = row_of(t) < ndb ? row_of(t) : 0;
            Operand<AR, P>::fetch_f32(static_cast<const float*>(dbase) + row * d, row_of(t) < ndb, raw);
        };
        fetch(t0);
        Operand<AR, P> r;
        r.split_f32(raw, h, role);
        for (int t = t0; t < t1; ++t) {
            fetch(t + 1 < t1 ? t + 1 : t);
            compute(r, t);
            r.split_f32(raw, h, role);
        }
    } else {
        auto get = [&](Operand<AR, P>& o, int t) {
            const int64_t row = row_of(t) < ndb ? row_of(t) : 0;
            o.load(dbase, row, row_of(t) < ndb, h, d, role);
        };
        Operand<AR, P> rn;
        get(rn, t0);
        for (int t = t0; t < t1; ++t) {
            const Operand<AR, P> r = rn;
            const int tn = t + 1 < t1 ? t + 1 : t;
            get(rn, tn);
            compute(r, t);
        }
    }
}

// Work item = (query group, database segment).  A query group is four query blocks of
// 32*QT queries, one per wave; the segment is a contiguous range of 32-row tiles.
// The number of segments follows the live query count (read on the device), so a
// shrinking frontier still spreads over the whole GPU; it is a multiple of 8 when
// possible so that each XCD keeps streaming the same eighth of the database through
// its own L2.  Every wave leaves one atomicMax per query and item.  With
// tile_best arithmetic the merged key names (score, tile) and recover_rows_kernel
// turns it into (score, row).
// Waves per SIMD the compiler must leave room for (register budget): three for the
// short bf16 contraction, whose database ring and accumulators otherwise land just
// above that budget; the split-fp32 and fp32 forms need their registers.
template <int AR, int P> constexpr int min_waves() { return AR == AR_BF16 && P <= 2 ? 3 : 1; }

template <int AR, int P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(min_waves<AR, P>())))
void nn_argmax_kernel(NNArgs a) {
    constexpr int QT = qt_of<AR, P>();
    constexpr bool TB = ArithTraits<AR>::tile_best;   // keys carry (score, tile), not (score, row)
    constexpr int QB = 32 * QT;          // queries per wave
    constexpr int LDS_TILES = (AR == AR_BF16 ? 3 * kStageTiles : 2) * 32 * lds_row_bytes<AR, P>();
    constexpr int LDS_RED = kWaves * QB * 8;
    __shared__ __attribute__((aligned(16))) char lds[LDS_TILES > LDS_RED ? LDS_TILES : LDS_RED];
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, so branches on it stay scalar
    int pair, bx, gx;   // pair, workgroup within the pair, workgroups per pair
    if (a.xcd_gx) {
        const int k = (int)blockIdx.x >> 3;
        gx = a.xcd_gx;
        bx = k % gx;
        pair = (int)(blockIdx.x & 7) + 8 * (k / gx);
        if (pair >= a.batch) return;
    } else {
        pair = blockIdx.y;
        bx = blockIdx.x;
        gx = gridDim.x;
    }
    const int n = __builtin_amdgcn_readfirstlane(a.dev_count ? a.dev_count[pair * a.count_stride] : a.host_count);
    const int ntiles = (a.ndb + 31) >> 5;
    const int nqt = (n + 31) >> 5;                        // query tiles
    const int qgroups = (nqt + kWaves * QT - 1) / (kWaves * QT);
    if (qgroups == 0 || ntiles == 0) return;
    int nsg = gx / qgroups;
    const int sg_cap = ntiles < kMaxSegGroups ? ntiles : kMaxSegGroups;
    nsg = nsg < 1 ? 1 : (nsg > sg_cap ? sg_cap : nsg);
    if (nsg >= 8) nsg &= ~7;
    const int items = qgroups * nsg;
    const void* qbase = pair_base<AR>(a.qmap, a.q_pair_elems, map_of(a.q_img, pair));
    const char* dbytes = static_cast<const char*>(pair_base<AR>(a.dbmap, a.db_pair_elems, map_of(a.db_img, pair)));
    const int rb = row_bytes<AR>(a.d);

    // query tile j of a wave is tile (tb + j*ts) of the query list
    auto load_queries = [&](Operand<AR, P> (&q)[QT], int tb, int ts, int nact) {
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            if (j < nact) {
                const int qp = (tb + j * ts) * 32 + jl;
                int64_t row = qp;
                bool valid = qp < n;
                if (valid && a.qsrc == Q_LIST) row = a.qlist[pair * a.qlist_stride + qp];
                valid = valid && row >= 0 && row < a.nq_rows;
                if constexpr (AR == AR_X3)
                    q[j].load_f32(static_cast<const float*>(qbase) + (valid ? row : 0) * a.d, valid, h, a.q_role);
                else
                    q[j].load(qbase, valid ? row : 0, valid, h, a.d, a.q_role);
            } else if constexpr (AR == AR_BF16) {
                q[j].load(qbase, 0, false, h, a.d, a.q_role);   // zero: the register stream runs every slot
            }
        }
    };
    auto finish = [&](const KeyBest<QT>& b, float (&sv)[QT], int (&rw)[QT]) {
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            sv[j] = __int_as_float(b.bk[j] & ~15);
            rw[j] = b.bt[j] >= 0 ? b.bt[j] * 32 + tile_row(15 - (b.bk[j] & 15), h) : -1;
        }
    };
    auto finish_exact = [&](const ExactBest<QT>& b, float (&sv)[QT], int (&rw)[QT]) {
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            sv[j] = b.bv[j];
            rw[j] = b.bx[j] >= 0 ? (b.bx[j] >> 4) * 32 + tile_row(b.bx[j] & 15, h) : -1;
        }
    };

    if (qgroups == 1 && nqt < kWaves) {
        // small frontier (fewer query tiles than waves, so some wave of the one query
        // group would sit idle): the four waves share each query block and split the
        // database four ways; query blocks are taken one after another
        const int cap = (ntiles + kWaves - 1) / kWaves < kMaxSegGroups ? (ntiles + kWaves - 1) / kWaves
                                                                       : kMaxSegGroups;
        const int ngroups = gx < cap ? gx : cap;
        const int nqb = (n + QB - 1) / QB;
        uint64_t* red = reinterpret_cast<uint64_t*>(lds);
        for (int item = bx; item < ngroups * nqb; item += gx) {
            const int qb = item / ngroups, grp = item - qb * ngroups;
            const int q0 = qb * QB;
            const int left = n - q0;
            const int nact = left >= QB ? QT : (left + 31) >> 5;
            Operand<AR, P> q[QT];
            load_queries(q, q0 >> 5, 1, nact);
            const int seg = grp * kWaves + wv, nseg = ngroups * kWaves;
            const int t0 = __builtin_amdgcn_readfirstlane((int)((int64_t)seg * ntiles / nseg));
            const int t1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(seg + 1) * ntiles / nseg));
            float sv[QT];
            int rw[QT];   // row, or tile with TB
            if constexpr (TB) {
                TileBest<QT> best;
                stream_direct<AR, P>(dbytes, t0, t1, a.ndb, q, nact, h, jl, a.d, a.db_role, best);
#pragma unroll
                for (int j = 0; j < QT; ++j) { sv[j] = best.bv[j]; rw[j] = best.bt[j]; }
            } else {
                KeyBest<QT> best;
                stream_direct<AR, P>(dbytes, t0, t1, a.ndb, q, nact, h, jl, a.d, a.db_role, best);
                finish(best, sv, rw);
                bool neg = false;
#pragma unroll
                for (int j = 0; j < QT; ++j) neg = neg || (j < nact && best.bk[j] < 0 && t0 < t1);
                if (__ballot(neg) != 0) {
                    ExactBest<QT> exact;
                    stream_direct<AR, P>(dbytes, t0, t1, a.ndb, q, nact, h, jl, a.d, a.db_role, exact);
                    finish_exact(exact, sv, rw);
                }
            }
#pragma unroll
            for (int j = 0; j < QT; ++j) {
                uint64_t key = rw[j] >= 0 ? pack_key(sv[j], (uint32_t)rw[j]) : 0;
                const uint64_t o = shfl_xor_u64(key, 32);
                key = o > key ? o : key;
                if (h == 0) red[wv * QB + j * 32 + jl] = j < nact ? key : 0;
            }
            __syncthreads();
            if (threadIdx.x < QB) {
                uint64_t key = red[threadIdx.x];
#pragma unroll
                for (int w = 1; w < kWaves; ++w) key = red[w * QB + threadIdx.x] > key ? red[w * QB + threadIdx.x] : key;
                const int qp = q0 + (int)threadIdx.x;
                if (qp < n && key != 0)
                    atomicMax(reinterpret_cast<unsigned long long*>(&a.keys[pair * a.keys_stride + qp]),
                              (unsigned long long)key);
            }
            __syncthreads();
        }
        return;
    }

    for (int item = bx; item < items; item += gx) {
        const int qg = item / nsg;
        const int sg = item - qg * nsg;
        // the query tiles are spread evenly over the groups; a group's tiles are dealt
        // round-robin to its waves (tile g0 + wv + kWaves*j)
        const int g0 = (int)((int64_t)qg * nqt / qgroups);
        const int g1 = (int)((int64_t)(qg + 1) * nqt / qgroups);
        const int nact = __builtin_amdgcn_readfirstlane(g0 + wv < g1 ? (g1 - g0 - wv + kWaves - 1) / kWaves : 0);

        Operand<AR, P> q[QT];
        load_queries(q, g0 + wv, kWaves, nact);
        // the segment bounds are wave-uniform: kept in scalar registers, the tile loop's
        // control and the tiles' base addresses stay off the vector ALUs
        const int t0 = __builtin_amdgcn_readfirstlane((int)((int64_t)sg * ntiles / nsg));
        const int t1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(sg + 1) * ntiles / nsg));

        // (score, row) -- or (score, tile) with TB -- per lane and query tile
        float sv[QT];
        int rw[QT];
        if constexpr (TB) {
            TileBest<QT> best;
            // segments without a ragged tile stream through registers, each wave on its
            // own (a wave short of query tiles multiplies zero operands in the empty
            // slots, whose keys are never written; a wave with none skips the stream);
            // the choice is the same for all four waves, as the staged path has barriers
            if ((int64_t)t1 * 32 <= a.ndb) {
                if (nact > 0) stream_regs<AR, P, 4>(dbytes, t0, t1, q, h, jl, a.d, best);
            } else {
                stream_db<AR, P>(dbytes, rb, t0, t1, a.ndb, lds, q, nact, h, jl, a.d, a.db_role, best);
            }
#pragma unroll
            for (int j = 0; j < QT; ++j) { sv[j] = best.bv[j]; rw[j] = best.bt[j]; }
        } else {
            KeyBest<QT> best;
            stream_db<AR, P>(dbytes, rb, t0, t1, a.ndb, lds, q, nact, h, jl, a.d, a.db_role, best);
            finish(best, sv, rw);
            bool neg = false;
#pragma unroll
            for (int j = 0; j < QT; ++j) neg = neg || (j < nact && best.bk[j] < 0);
            if (__syncthreads_or(neg)) {
                // some lane's best score is negative, where float bits do not order as
                // integers: the workgroup streams its segment again with the exact comparison
                ExactBest<QT> exact;
                stream_db<AR, P>(dbytes, rb, t0, t1, a.ndb, lds, q, nact, h, jl, a.d, a.db_role, exact);
                finish_exact(exact, sv, rw);
            }
        }

        // merge the two lane halves of each query, then across items with atomicMax
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            uint64_t key = rw[j] >= 0 ? pack_key(sv[j], (uint32_t)rw[j]) : 0;
            const uint64_t o = shfl_xor_u64(key, 32);
            key = o > key ? o : key;
            const int qp = (g0 + wv + j * kWaves) * 32 + jl;
            if (h == 0 && j < nact && qp < n && key != 0)
                atomicMax(reinterpret_cast<unsigned long long*>(&a.keys[pair * a.keys_stride + qp]),
                          (unsigned long long)key);
        }
    }
}

// (score, tile) -> (score, row): one query tile per workgroup; each wave takes 8 of
// its 32 queries.  For query c the wave loads the 32 rows of c's tile as the A
// operand and multiplies them with the query block exactly as the streaming pass
// did (same instruction, same operand layout, same step order), so column c holds
// bitwise the scores that were compared there; the lowest row whose trunc4 score
// equals the key's score is c's NN.  Keys are rewritten in place.
template <int AR, int P>
__global__ __launch_bounds__(kThreads) void recover_rows_kernel(NNArgs a) {
    constexpr int CPW = 32 / kWaves;   // queries resolved per wave
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform, so branches on it stay scalar
    const int pair = blockIdx.y;
    const int n = __builtin_amdgcn_readfirstlane(a.dev_count ? a.dev_count[pair * a.count_stride] : a.host_count);
    const int nqt = (n + 31) >> 5;
    const void* qbase = pair_base<AR>(a.qmap, a.q_pair_elems, map_of(a.q_img, pair));
    const void* dbase = pair_base<AR>(a.dbmap, a.db_pair_elems, map_of(a.db_img, pair));
    uint64_t* keys = a.keys + pair * a.keys_stride;
    for (int g = blockIdx.x; g < nqt; g += gridDim.x) {
        const int qp = g * 32 + jl;
        int64_t row = qp;
        bool valid = qp < n;
        if (valid && a.qsrc == Q_LIST) row = a.qlist[pair * a.qlist_stride + qp];
        valid = valid && row >= 0 && row < a.nq_rows;
        Operand<AR, P> q;
        q.load(qbase, valid ? row : 0, valid, h, a.d, a.q_role);
        // this lane's query key; only columns 8*wv.. are read back below, and only this
        // wave rewrites them, after the read
        const uint64_t key = qp < n ? keys[qp] : 0;
        Operand<AR, P> r[CPW];
        int tile[CPW];
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            const uint64_t kc = shfl_u64(key, CPW * wv + k);
            tile[k] = kc ? (int)~(uint32_t)kc : -1;
            const int64_t drow = (int64_t)tile[k] * 32 + jl;
            const bool ok = tile[k] >= 0 && drow < a.ndb;
            r[k].load(dbase, ok ? drow : 0, ok, h, a.d, a.db_role);
        }
        uint64_t out = 0;
#pragma unroll
        for (int k = 0; k < CPW; ++k) {
            const int c = CPW * wv + k;
            const uint64_t kc = shfl_u64(key, c);
            const float best = from_ordered((uint32_t)(kc >> 32));
            f32x16 acc = {};
            acc = r[k].mfma(q, acc);
            int found = INT_MAX;
#pragma unroll
            for (int v = 15; v >= 0; --v) {
                const int rr = tile[k] * 32 + tile_row(v, h);
                if (trunc4(acc[v]) == best && rr < a.ndb) found = rr;
            }
            const int o = __shfl_xor(found, 32);
            found = o < found ? o : found;
            if (jl == c) out = (kc != 0 && found != INT_MAX) ? pack_key(best, (uint32_t)found) : 0;
        }
        if (h == 0 && qp < n && jl >= CPW * wv && jl < CPW * (wv + 1)) keys[qp] = out;
    }
}

// ---------------------------------------------------------------------------- fused row + column argmax

// Brute-force reciprocal NN needs both nearest-neighbour maps of one similarity
// matrix: NN(a_i, b) over its rows and NN(b_k, a) over its columns ("MASt3R
// dissection", section 1 diagram: the match set needs both directions; section 3
// "Napkin Formula").  rowcol_argmax_kernel computes every 32x32 similarity tile once
// and reduces it both ways:
//  - rows (queries = pixels of a, held as MFMA B operands): the tile-level running
//    maximum of TileBest (best compared score, first b tile reaching it), merged
//    across database segments by atomicMax on (score, ~tile) keys and resolved to a
//    row by recover_rows_kernel;
//  - columns (pixels of b, streamed as MFMA A operands): per b tile, each lane's
//    maximum over the wave's query tiles (in-lane, a max3 fold), then a transpose
//    through LDS and a 16-value maximum per row (one lane pair per row of the tile),
//    then a maximum over the workgroup's waves and one atomicMax per b row and
//    workgroup on (score, ~query block) keys, a query block being the 256
//    consecutive query pixels of one wave.  The column recovery (rows bucketed by
//    winning block, recover_cols_gathered_kernel) resolves each winning block to the
//    lowest query row of the winning score.
// Both directions compare scores after clearing their 4 low bits, lowest index on
// ties, exactly like nn_argmax_kernel, so the results equal two separate searches.
// The b tiles of a workgroup's segment pass through a two-group LDS ring, copied
// straight from global memory into LDS (global_load_lds, no registers) one group of
// kRcFlush tiles ahead; the barrier that publishes a group's wave maxima also
// publishes the next group's copy.  The matrix work is half that of two searches; the
// vector work (a tile-level row maximum and a column fold for every score) is about
// the same, and it bounds the kernel on this chip.
constexpr int kRcWaves = 8;                 // waves per workgroup (two per SIMD)
constexpr int kRcThreads = 64 * kRcWaves;
constexpr int kRcQT = 8;                    // query tiles per wave (one query block)
constexpr int kRcGroupTiles = kRcWaves * kRcQT;
constexpr int kRcFlush = 8;                 // b tiles per column merge (one barrier each)
constexpr int kRcPad = 36;                  // floats per row of the transpose area (16-byte rows, no write conflicts)
constexpr int kRcMaxTileBytes = 32 * 64;    // a 32-row b tile of bf16 rows, d <= 32
constexpr uint32_t kWaitVm0 = 0x0F70;       // s_waitcnt vmcnt(0) (expcnt, lgkmcnt at their maximum)

typedef const void __attribute__((address_space(1)))* gptr_t;
typedef void __attribute__((address_space(3)))* lptr_t;

struct RowColArgs {
    const void* amap;        // [batch][na][d] bf16: queries (rows of the similarity)
    const void* bmap;        // [batch][nb][d] bf16: streamed (columns)
    int64_t a_pair_elems, b_pair_elems;
    int32_t na, nb, d;
    int32_t nsg;             // b segments per query group
    uint64_t* keys_ab;       // [batch][na]: (score, ~b tile)
    uint64_t* keys_ba;       // [batch][nb]: (score, ~query block)
};

template <int P>
__global__ __launch_bounds__(kRcThreads) void rowcol_argmax_kernel(RowColArgs a) {
    using Op = Operand<AR_BF16, P>;
    __shared__ __attribute__((aligned(16))) float tr[kRcWaves][32 * kRcPad];   // per-wave transpose
    __shared__ float mg[2 * kRcFlush + 1][kRcWaves][32];   // wave maxima, two sets (+ a discard slot)
    __shared__ __attribute__((aligned(16))) char ring[2][kRcFlush * kRcMaxTileBytes];   // b tiles, two groups
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.y;
    const int na = a.na, nb = a.nb, d = a.d;
    const int nqt = (na + 31) >> 5;
    const int ntiles = (nb + 31) >> 5;
    const int qgroups = (nqt + kRcGroupTiles - 1) / kRcGroupTiles;
    const int nsg = a.nsg;
    const int items = qgroups * nsg;
    const void* abase = static_cast<const uint16_t*>(a.amap) + pair * a.a_pair_elems;
    const char* bbytes = reinterpret_cast<const char*>(static_cast<const uint16_t*>(a.bmap) + pair * a.b_pair_elems);
    uint64_t* keys_ab = a.keys_ab + (int64_t)pair * na;
    uint64_t* keys_ba = a.keys_ba + (int64_t)pair * nb;
    int off[P];
    Op::db_offsets(jl, h, d, off);
    const int64_t tile_bytes = (int64_t)64 * d;   // 32 rows of 2d bytes
    float* trw = tr[wv];
    int gc = 0;   // merge sets used so far (alternating halves of mg)

    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int qg = item / nsg;
        const int sg = item - qg * nsg;
        const int tq0 = qg * kRcGroupTiles + wv * kRcQT;               // this wave's first query tile
        const int nact = nqt - tq0 >= kRcQT ? kRcQT : (nqt - tq0 > 0 ? nqt - tq0 : 0);
        const int qvalid_last = na - (tq0 + kRcQT - 1) * 32;            // valid lanes of the last tile
        const bool full = nact == kRcQT && qvalid_last >= 32;           // no partial query tile
        Op q[kRcQT];
#pragma unroll
        for (int j = 0; j < kRcQT; ++j) {
            const int qp = (tq0 + j) * 32 + jl;
            const bool valid = j < nact && qp < na;
            q[j].load(abase, valid ? qp : 0, valid, h, d, 1);
        }
        // segments are whole groups of kRcFlush tiles (the host keeps nsg <= groups), so
        // every group a segment visits is one of the map's fixed groups [8k, 8k + 8)
        const int ngroups = (ntiles + kRcFlush - 1) / kRcFlush;
        const int t0 = (int)((int64_t)sg * ngroups / nsg) * kRcFlush;
        const int t1e = (int)((int64_t)(sg + 1) * ngroups / nsg) * kRcFlush;
        const int t1 = t1e < ntiles ? t1e : ntiles;
        GroupBest<kRcQT> best;

        // b tiles [tg, tend) are copied into ring set `set` by the workgroup, straight
        // from global memory into LDS (no registers), 16 bytes per lane: the group's
        // real rows are contiguous in memory and in the set; lanes past them repeat the
        // last chunk into the unused rest of the set
        auto load_group = [&](int tg, int tend, int set) {
            const int rows = (tend * 32 < nb ? tend * 32 : nb) - tg * 32;
            const int nch = rows * (2 * d) / 16;
            const char* src = bbytes + (int64_t)tg * tile_bytes;
            for (int i = wv; i * 64 < nch; i += kRcWaves) {
                const int ch = i * 64 + lane < nch ? i * 64 + lane : nch - 1;
                __builtin_amdgcn_global_load_lds((gptr_t)(src + (int64_t)ch * 16), (lptr_t)(&ring[set][i * 1024]), 16,
                                                 0, 0);
            }
        };
        // column values of tile t (the lane's maximum over its valid queries, rows
        // (h, v)) -> the wave's maximum per row, through the transpose area, into merge
        // slot k of the current set
        auto column_out = [&](const float (&c)[16], int set, int k) {
#pragma unroll
            for (int v = 0; v < 16; ++v) trw[(h * 16 + v) * kRcPad + jl] = c[v];
            const int rr = lane >> 1;
            const float4* src = reinterpret_cast<const float4*>(trw + rr * kRcPad + (lane & 1) * 16);
            const float4 y0 = src[0], y1 = src[1], y2 = src[2], y3 = src[3];
            auto mx3 = [](float p, float q_, float s_) {
                return __builtin_elementwise_maximum(__builtin_elementwise_maximum(p, q_), s_);
            };
            float m = mx3(mx3(y0.x, y0.y, y0.z), mx3(y0.w, y1.x, y1.y), mx3(y1.z, y1.w, y2.x));
            m = mx3(m, mx3(y2.y, y2.z, y2.w), mx3(y3.x, y3.y, y3.z));
            m = __builtin_elementwise_maximum(m, y3.w);
            m = __builtin_elementwise_maximum(m, __shfl_xor(m, 1));
            if ((lane & 1) == 0) mg[set + k][wv][tile_row(rr & 15, rr >> 4)] = m;
        };
        // after a group of tiles: merge the waves (lowest block on equal compared
        // scores) and leave one atomic per b row and workgroup
        auto merge = [&](int set, int tg, int tend) {
            __syncthreads();
            if ((int)threadIdx.x < kRcFlush * 32) {
                const int k = threadIdx.x >> 5, rw = threadIdx.x & 31;
                const int t = tg + k;
                if (t < tend) {
                    float bs = -INFINITY;
                    int bw = -1;
#pragma unroll
                    for (int w = 0; w < kRcWaves; ++w) {
                        const float x = trunc4(mg[set + k][w][rw]);
                        if (x > bs) { bs = x; bw = w; }
                    }
                    const int row = t * 32 + rw;
                    if (bw >= 0 && row < nb)
                        atomicMax(reinterpret_cast<unsigned long long*>(&keys_ba[row]),
                                  (unsigned long long)(((uint64_t)ordered_bits(bs) << 32) |
                                                       (uint64_t)(~(uint32_t)(qg * kRcWaves + bw))));
                }
            }
        };
        // the segment in groups of kRcFlush tiles: group g + 1 is copied into LDS while
        // group g is multiplied; one barrier per group publishes the copy and the wave
        // maxima.  FAST: every query tile of the wave full and no ragged b tile
        // (straight-line code, query tiles in pairs with one max3 per column value).
        auto stream = [&](auto fast) {
            constexpr bool FAST = decltype(fast)::value;
            if (t0 < t1) {
                load_group(t0, t0 + kRcFlush < t1 ? t0 + kRcFlush : t1, gc & 1);
                __builtin_amdgcn_s_waitcnt(kWaitVm0);
                __syncthreads();
            }
            for (int tg = t0; tg < t1; tg += kRcFlush, ++gc) {
                const int tend = tg + kRcFlush < t1 ? tg + kRcFlush : t1;
                const int set = gc & 1;
                if (tend < t1) load_group(tend, tend + kRcFlush < t1 ? tend + kRcFlush : t1, set ^ 1);
                if constexpr (FAST) {
                    // units of two query tiles; the epilogue of each unit (rows of both,
                    // and the column fold) runs one unit behind its products, between the
                    // products of the next unit, which also keeps one unit's products live
                    // at a time; the column values of a tile leave through the transpose
                    // after its last unit's epilogue.  The group starts with a stand-in
                    // unit of -inf scores (it changes no row state) whose column output
                    // goes to the discard slot.  The b operand is read from LDS one tile
                    // ahead (the whole group is in the ring; the read past its last tile
                    // stays inside the set).
                    f32x16 p0, p1;
#pragma unroll
                    for (int v = 0; v < 16; ++v) { p0[v] = -INFINITY; p1[v] = -INFINITY; }
                    float c[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) c[v] = -INFINITY;
                    auto fold = [&](const f32x16& y0, const f32x16& y1, int tt, int j) {
                        best.template tile<false>(y0, tt, h, nb, j);
                        best.template tile<false>(y1, tt, h, nb, j + 1);
                        if (j == 0) {
#pragma unroll
                            for (int v = 0; v < 16; ++v) c[v] = __builtin_elementwise_maximum(y0[v], y1[v]);
                        } else {
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                c[v] = __builtin_elementwise_maximum(__builtin_elementwise_maximum(c[v], y0[v]), y1[v]);
                        }
                    };
                    Op nxt;
                    nxt.load_db(&ring[set][0], off);
                    for (int t = tg; t < tend; ++t) {
                        const Op cur = nxt;
                        nxt.load_db(&ring[set][(t + 1 - tg < kRcFlush ? t + 1 - tg : 0) * tile_bytes], off);
#pragma unroll
                        for (int j = 0; j < kRcQT; j += 2) {
                            const f32x16 x0 = cur.mfma(q[j], f32x16{});
                            const f32x16 x1 = cur.mfma(q[j + 1], f32x16{});
                            if (j == 0) {
                                // the previous tile's last unit, then its column output
                                fold(p0, p1, t - 1, kRcQT - 2);
                                column_out(c, t == tg ? 2 * kRcFlush : set * kRcFlush + (t - 1 - tg), 0);
                                interleave_mfma_valu<2 * P, 14>();
                            } else {
                                fold(p0, p1, t, j - 2);
                                interleave_mfma_valu<2 * P, 10>();
                            }
                            __builtin_amdgcn_sched_barrier(0);
                            p0 = x0;
                            p1 = x1;
                        }
                    }
                    fold(p0, p1, tend - 1, kRcQT - 2);
                    column_out(c, set * kRcFlush + (tend - 1 - tg), 0);
                } else {
                for (int t = tg; t < tend; ++t) {
                    Op cur;
                    cur.load_db(&ring[set][(t - tg) * tile_bytes], off);
                    float c[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) c[v] = -INFINITY;
                    const bool ragged = (t + 1) * 32 > nb;
#pragma unroll
                    for (int j = 0; j < kRcQT; ++j) {
                        if (j < nact) {
                            const f32x16 x = cur.mfma(q[j], f32x16{});
                            best.step(x, t, h, nb, j, ragged);
                            // queries past na hold zero operands: they take no part in the columns
                            const bool qok = (tq0 + j) * 32 + jl < na;
#pragma unroll
                            for (int v = 0; v < 16; ++v)
                                c[v] = qok ? __builtin_elementwise_maximum(c[v], x[v]) : c[v];
                        }
                    }
                    column_out(c, set * kRcFlush, t - tg);
                }
                }
                best.close(tg / kRcFlush);              // rows: the group's maxima
                __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's copies of the next group
                merge(set * kRcFlush, tg, tend);        // barrier, then the wave maxima
            }
        };
        if (full && t1 * 32 <= nb) stream(std::true_type{});
        else stream(std::false_type{});

        // rows: merge the lane halves, one atomic per query and item
#pragma unroll
        for (int j = 0; j < kRcQT; ++j) {
            uint64_t key = best.bt[j] >= 0 ? pack_key(best.bv[j], (uint32_t)best.bt[j]) : 0;
            const uint64_t o = shfl_xor_u64(key, 32);
            key = o > key ? o : key;
            const int qp = (tq0 + j) * 32 + jl;
            if (h == 0 && j < nact && qp < na && key != 0)
                atomicMax(reinterpret_cast<unsigned long long*>(&keys_ab[qp]), (unsigned long long)key);
        }
    }
}

// Recoveries of the fused pass by bucket.  Each direction's keys name a bucket in their
// low word (a query block for the columns, a group of b tiles for the rows); the
// entries are gathered into one list per bucket (count, prefix, scatter), then the
// bucket's shared operands are loaded once and compared with every gathered entry.
// A gathered 32-entry tile is an operand of the same instruction, with the same
// operand layout and step order as the fused pass (an output element depends only on
// its row and column operands, not on their places in the tile), so the scores are
// bitwise those that were compared.
struct Buckets {
    const uint64_t* keys;   // [batch][n] (score, ~bucket), 0 for none
    int64_t n;
    int32_t* cnt;     // [batch][nbins] entries per bucket
    int32_t* pos;     // [batch][nbins] prefix sums, then (after the scatter) end offsets
    int32_t* list;    // [batch][n] entry ids grouped by bucket
    int32_t nbins;
};

// Counting and scattering run per chunk of kBucketChunk rows (one workgroup of 256
// threads, kBucketChunk / 256 rows per thread).  With at most kBucketBins blocks the
// chunk's histogram is kept in LDS and the workgroup leaves one global atomic per
// non-empty block (same-address global atomics serialise); otherwise every row adds
// to the global count itself.
constexpr int kBucketChunk = 2048;
constexpr int kBucketBins = 8192;

// Both directions in one launch: blockIdx.z selects the bucket set (0 = b0, 1 = b1).
__global__ __launch_bounds__(256) void bucket_count_kernel(Buckets b0, Buckets b1) {
    __shared__ int32_t hist[kBucketBins];
    const Buckets c = blockIdx.z ? b1 : b0;
    if ((int64_t)blockIdx.x * kBucketChunk >= c.n) return;
    const int pair = blockIdx.y;
    const uint64_t* keys = c.keys + (int64_t)pair * c.n;
    int32_t* cnt = c.cnt + (int64_t)pair * c.nbins;
    const bool local = c.nbins <= kBucketBins;
    if (local) {
        for (int i = threadIdx.x; i < c.nbins; i += 256) hist[i] = 0;
        __syncthreads();
    }
    const int64_t r0 = (int64_t)blockIdx.x * kBucketChunk;
#pragma unroll
    for (int e = 0; e < kBucketChunk / 256; ++e) {
        const int64_t i = r0 + e * 256 + threadIdx.x;
        const uint64_t k = i < c.n ? keys[i] : 0;
        const uint32_t b = ~(uint32_t)k;
        if (k && b < (uint32_t)c.nbins) {
            if (local) atomicAdd(&hist[b], 1);
            else atomicAdd(&cnt[b], 1);
        }
    }
    if (local) {
        __syncthreads();
        for (int i = threadIdx.x; i < c.nbins; i += 256)
            if (hist[i]) atomicAdd(&cnt[i], hist[i]);
    }
}

// exclusive prefix of the counts, one workgroup of 1024 threads per pair, 1024 counts
// per step
__global__ __launch_bounds__(1024) void bucket_scan_kernel(Buckets b0, Buckets b1) {
    __shared__ int32_t part[1024 / 64];
    const Buckets c = blockIdx.y ? b1 : b0;
    const int pair = blockIdx.x;
    const int32_t* cnt = c.cnt + (int64_t)pair * c.nbins;
    int32_t* pos = c.pos + (int64_t)pair * c.nbins;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    int32_t carry = 0;
    for (int base = 0; base < c.nbins; base += 1024) {
        const int i = base + (int)threadIdx.x;
        const int32_t v = i < c.nbins ? cnt[i] : 0;
        int32_t x = v;   // inclusive scan within the wave
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
            const int32_t o = __shfl_up(x, m);
            if (lane >= m) x += o;
        }
        if (lane == 63) part[wv] = x;
        __syncthreads();
        int32_t before = carry;
        for (int w = 0; w < wv; ++w) before += part[w];
        int32_t total = 0;
        for (int w = 0; w < 1024 / 64; ++w) total += part[w];
        if (i < c.nbins) pos[i] = before + x - v;
        carry += total;
        __syncthreads();
    }
}

// rows -> their block's list; with the LDS histogram a row's place is its block's base
// for this chunk (one global atomic per non-empty block) plus its rank in the chunk
__global__ __launch_bounds__(256) void bucket_scatter_kernel(Buckets b0, Buckets b1) {
    __shared__ int32_t hist[kBucketBins];
    const Buckets c = blockIdx.z ? b1 : b0;
    if ((int64_t)blockIdx.x * kBucketChunk >= c.n) return;
    const int pair = blockIdx.y;
    const uint64_t* keys = c.keys + (int64_t)pair * c.n;
    int32_t* pos = c.pos + (int64_t)pair * c.nbins;
    int32_t* list = c.list + (int64_t)pair * c.n;
    const int64_t r0 = (int64_t)blockIdx.x * kBucketChunk;
    if (c.nbins > kBucketBins) {
#pragma unroll
        for (int e = 0; e < kBucketChunk / 256; ++e) {
            const int64_t i = r0 + e * 256 + threadIdx.x;
            const uint64_t k = i < c.n ? keys[i] : 0;
            const uint32_t b = ~(uint32_t)k;
            if (k && b < (uint32_t)c.nbins) list[atomicAdd(&pos[b], 1)] = (int32_t)i;
        }
        return;
    }
    for (int i = threadIdx.x; i < c.nbins; i += 256) hist[i] = 0;
    __syncthreads();
    int bk[kBucketChunk / 256], rk[kBucketChunk / 256];
#pragma unroll
    for (int e = 0; e < kBucketChunk / 256; ++e) {
        const int64_t i = r0 + e * 256 + threadIdx.x;
        const uint64_t k = i < c.n ? keys[i] : 0;
        const uint32_t b = ~(uint32_t)k;
        bk[e] = (k && b < (uint32_t)c.nbins) ? (int)b : -1;
        rk[e] = bk[e] >= 0 ? atomicAdd(&hist[bk[e]], 1) : 0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < c.nbins; i += 256)
        if (hist[i]) hist[i] = atomicAdd(&pos[i], hist[i]);   // this chunk's base in block i's list
    __syncthreads();
#pragma unroll
    for (int e = 0; e < kBucketChunk / 256; ++e)
        if (bk[e] >= 0) list[hist[bk[e]] + rk[e]] = (int32_t)(r0 + e * 256 + threadIdx.x);
}

// Columns: one workgroup per query block; its waves share the block's gathered b rows,
// each row taking the lowest query of the block whose compared score equals its key's.
template <int P>
__device__ __forceinline__ void recover_cols_gathered_body(RowColArgs a, const Buckets& c) {
    using Op = Operand<AR_BF16, P>;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.y;
    const int na = a.na, nb = a.nb, d = a.d;
    const int nqt = (na + 31) >> 5;
    const void* abase = static_cast<const uint16_t*>(a.amap) + pair * a.a_pair_elems;
    const void* bbase = static_cast<const uint16_t*>(a.bmap) + pair * a.b_pair_elems;
    uint64_t* keys_ba = a.keys_ba + (int64_t)pair * nb;
    const int32_t* cnt = c.cnt + (int64_t)pair * c.nbins;
    const int32_t* pos = c.pos + (int64_t)pair * c.nbins;
    const int32_t* list = c.list + (int64_t)pair * nb;
    for (int blk = blockIdx.x; blk < c.nbins; blk += gridDim.x) {
        const int n = cnt[blk];
        if (n == 0) continue;
        const int begin = pos[blk] - n;   // the scatter advanced pos to the block's end
        const int tq0 = blk * kRcQT;
        Op qb[kRcQT];
#pragma unroll
        for (int j = 0; j < kRcQT; ++j) {
            const int qp = (tq0 + j) * 32 + jl;
            qb[j].load(abase, qp < na ? qp : 0, qp < na, h, d, 1);
        }
        for (int g = wv; g * 32 < n; g += kWaves) {
            // this lane's A row (tile position jl) with its key's score; the scores of
            // the rows (h, v) whose results the lane sees come from the lanes holding them
            const int ia = g * 32 + jl;
            const int arow = ia < n ? list[begin + ia] : -1;
            Op r;
            r.load(bbase, arow >= 0 ? arow : 0, arow >= 0, h, d, 2);
            const float sc_lane = arow >= 0 ? from_ordered((uint32_t)(keys_ba[arow] >> 32)) : 0.0f;
            f32x16 sc;
            i32x16 found;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                sc[v] = __shfl(sc_lane, tile_row(v, h));
                found[v] = g * 32 + tile_row(v, h) < n ? INT_MAX : INT_MIN;   // INT_MIN: no row there
            }
#pragma unroll
            for (int j = 0; j < kRcQT; ++j) {
                if (tq0 + j >= nqt) break;
                const int qp = (tq0 + j) * 32 + jl;
                const f32x16 x = r.mfma(qb[j], f32x16{});
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    if (qp < na && trunc4(x[v]) == sc[v] && qp < found[v]) found[v] = qp;
            }
            // lowest query over the 32 lanes of each half; lane (h, jl < 16) writes the
            // gathered row at (h, v = jl)
            int mine = INT_MAX;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                int f = found[v];
#pragma unroll
                for (int m = 16; m >= 1; m >>= 1) {
                    const int o = __shfl_xor(f, m);
                    f = o < f ? o : f;
                }
                if (jl == v) mine = f;
            }
            const int myrow = __shfl(arow, tile_row(jl & 15, h));
            if (jl < 16 && myrow >= 0) {
                const uint64_t k = keys_ba[myrow];
                keys_ba[myrow] = mine != INT_MAX ? pack_key(from_ordered((uint32_t)(k >> 32)), (uint32_t)mine) : 0;
            }
        }
    }
}

// Rows: one workgroup per group g of b tiles (the tiles [g * kRcFlush, g * kRcFlush +
// kRcFlush) of the map).  Each wave loads the group's tiles once as A operands and
// takes every fourth 32-query tile of the gathered queries as B operands; each query
// takes the lowest row of the group whose compared score equals its key's.
template <int P>
__device__ __forceinline__ void recover_rows_grouped_body(RowColArgs a, const Buckets& c) {
    using Op = Operand<AR_BF16, P>;
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.y;
    const int na = a.na, nb = a.nb, d = a.d;
    const int ntiles = (nb + 31) >> 5;
    const void* abase = static_cast<const uint16_t*>(a.amap) + pair * a.a_pair_elems;
    const void* bbase = static_cast<const uint16_t*>(a.bmap) + pair * a.b_pair_elems;
    uint64_t* keys_ab = a.keys_ab + (int64_t)pair * na;
    const int32_t* cnt = c.cnt + (int64_t)pair * c.nbins;
    const int32_t* pos = c.pos + (int64_t)pair * c.nbins;
    const int32_t* list = c.list + (int64_t)pair * na;
    for (int g = blockIdx.x; g < c.nbins; g += gridDim.x) {
        const int n = cnt[g];
        if (n <= wv * 32) continue;   // no query tile for this wave
        const int begin = pos[g] - n;
        const int g0 = g * kRcFlush;                                       // the group's first tile
        const int ng = ntiles - g0 < kRcFlush ? ntiles - g0 : kRcFlush;   // tiles of the group
        Op bt[kRcFlush];
#pragma unroll
        for (int k = 0; k < kRcFlush; ++k) {
            const int row = (g0 + k) * 32 + jl;
            bt[k].load(bbase, row < nb ? row : 0, k < ng && row < nb, h, d, 2);
        }
        for (int q0 = wv * 32; q0 < n; q0 += kWaves * 32) {
            const int iq = q0 + jl;
            const int qrow = iq < n ? list[begin + iq] : -1;
            Op qo;
            qo.load(abase, qrow >= 0 ? qrow : 0, qrow >= 0, h, d, 1);
            const float sc = qrow >= 0 ? from_ordered((uint32_t)(keys_ab[qrow] >> 32)) : 0.0f;
            int found = INT_MAX;
#pragma unroll
            for (int k = 0; k < kRcFlush; ++k) {
                if (k >= ng) break;
                const f32x16 x = bt[k].mfma(qo, f32x16{});
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int row = (g0 + k) * 32 + tile_row(v, h);
                    if (row < nb && trunc4(x[v]) == sc && row < found) found = row;
                }
            }
            const int o = __shfl_xor(found, 32);
            found = o < found ? o : found;
            if (h == 0 && qrow >= 0) keys_ab[qrow] = found != INT_MAX ? pack_key(sc, (uint32_t)found) : 0;
        }
    }
}

// Both recoveries of the fused pass in one launch: blockIdx.z = 0 the rows (a workgroup
// per group of b tiles), 1 the columns (a workgroup per query block), so the two
// overlap on the GPU.
template <int P>
__global__ __launch_bounds__(kThreads) void recover_rowcol_kernel(RowColArgs a, Buckets rows, Buckets cols) {
    if (blockIdx.z == 0) recover_rows_grouped_body<P>(a, rows);
    else recover_cols_gathered_body<P>(a, cols);
}

// ---------------------------------------------------------------------------- pointmaps

// Nearest neighbours of 3D points ("DUSt3R and MASt3R explained", the paragraph on
// recovering the cameras: two pixels correspond when their predicted 3D points are
// nearest neighbours in the shared frame).  d <= 4 is too short for the matrix cores,
// and the expanded form 2<x,y> - |y|^2 that would suit them cancels badly for points
// far from the origin, so the distance is computed directly on the VALU.
constexpr int kMaxPointD = 4;
constexpr int kPointQPL = 2;      // queries per lane
constexpr int kPointGroup = 16;   // database points per tracked group

typedef const float __attribute__((address_space(4))) cfloat;   // read through the scalar cache

// Squared distance with a fixed operation order and rounding (no contraction or
// reassociation): the search and the row recovery compute it bitwise alike.
template <int D, class T>
__device__ __forceinline__ float point_dist2(const float (&x)[D], const T* p) {
    float t = __fsub_rn(x[0], p[0]);
    float acc = __fmul_rn(t, t);
#pragma unroll
    for (int c = 1; c < D; ++c) {
        t = __fsub_rn(x[c], p[c]);
        acc = __fmaf_rn(t, t, acc);
    }
    return acc;
}

// Work item = (block of 128 queries, segment of database points), one per wave; waves
// never synchronise.  A lane holds two queries; the group of 16 database points it
// compares them with is uniform across the wave, so it comes through scalar loads
// and enters the VALU as scalar operands.  Per query and group a minimum tree folds
// the running best; the lane remembers the first group that reached it and, at the
// end of the segment, recomputes that group to find the lowest row at that
// distance.  Items merge with atomicMax on (ordered(-dist2), ~row) keys.  The number
// of segments follows the live query count (read on the device), a multiple of 8
// when possible so that each XCD keeps the same eighth of the database in its L2.
template <int D>
__global__ __launch_bounds__(kThreads) void point_nn_kernel(NNArgs a) {
    constexpr int QW = 64 * kPointQPL;   // queries per wave
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.y;
    const int n = __builtin_amdgcn_readfirstlane(a.dev_count ? a.dev_count[pair * a.count_stride] : a.host_count);
    const int ndb = a.ndb;
    if (n <= 0 || ndb <= 0) return;
    const int nqb = (n + QW - 1) / QW;
    const int waves = (int)gridDim.x * kWaves;
    const int seg_cap = ndb / 256 > 1 ? ndb / 256 : 1;        // segments of at least 256 points
    int nseg = waves / nqb;
    nseg = nseg < 1 ? 1 : (nseg > seg_cap ? seg_cap : nseg);
    if (nseg >= 8) nseg &= ~7;
    const float* qbase = static_cast<const float*>(a.qmap) + map_of(a.q_img, pair) * a.q_pair_elems;
    const float* dbase = static_cast<const float*>(a.dbmap) + map_of(a.db_img, pair) * a.db_pair_elems;
    uint64_t* keys = a.keys + pair * a.keys_stride;

    // consecutive workgroups take consecutive items, so item % 8 (the segment's XCD
    // share when nseg is a multiple of 8) follows blockIdx.x % 8
    for (int item = wv * (int)gridDim.x + (int)blockIdx.x; item < nqb * nseg; item += waves) {
        const int qb = item / nseg, sg = item - qb * nseg;
        const int p0 = (int)((int64_t)sg * ndb / nseg), p1 = (int)((int64_t)(sg + 1) * ndb / nseg);
        float x[kPointQPL][D], bv[kPointQPL];
        int qp[kPointQPL], bg[kPointQPL];
#pragma unroll
        for (int j = 0; j < kPointQPL; ++j) {
            qp[j] = qb * QW + j * 64 + lane;
            int64_t row = qp[j];
            bool valid = qp[j] < n;
            if (valid && a.qsrc == Q_LIST) row = a.qlist[pair * a.qlist_stride + qp[j]];
            valid = valid && row >= 0 && row < a.nq_rows;
#pragma unroll
            for (int c = 0; c < D; ++c) x[j][c] = valid ? qbase[row * D + c] : 0.0f;
            bv[j] = INFINITY;
            bg[j] = -1;
        }
        auto group = [&](int g, const auto* P, int npts) {
#pragma unroll
            for (int j = 0; j < kPointQPL; ++j) {
                float dd[kPointGroup];
#pragma unroll
                for (int k = 0; k < kPointGroup; ++k) {
                    dd[k] = point_dist2<D>(x[j], P + k * D);
                    if (npts < kPointGroup && k >= npts) dd[k] = INFINITY;
                }
                auto mn3 = [](float u, float v, float w) {
                    return __builtin_elementwise_minimum(__builtin_elementwise_minimum(u, v), w);
                };
                const float m0 = mn3(dd[0], dd[1], dd[2]), m1 = mn3(dd[3], dd[4], dd[5]);
                const float m2 = mn3(dd[6], dd[7], dd[8]), m3 = mn3(dd[9], dd[10], dd[11]);
                const float m4 = mn3(dd[12], dd[13], dd[14]), m5 = mn3(dd[15], bv[j], m0);
                const float m = mn3(mn3(m1, m2, m3), m4, m5);
                bg[j] = m != bv[j] ? g : bg[j];     // strictly nearer: the earliest group wins ties
                bv[j] = m;
            }
        };
        int g = p0;
        for (; g + kPointGroup <= p1; g += kPointGroup)
            group(g, (const cfloat*)(dbase + (int64_t)g * D), kPointGroup);
        if (g < p1) {
            // the last, partial group: its loads stay inside the segment (the first
            // point stands in for the missing ones, whose distances are masked)
            const int npts = p1 - g;
            float P[kPointGroup * D];
#pragma unroll
            for (int k = 0; k < kPointGroup; ++k)
#pragma unroll
                for (int c = 0; c < D; ++c) P[k * D + c] = dbase[(int64_t)(k < npts ? g + k : g) * D + c];
            group(g, P, npts);
        }
        // the lowest row of the remembered group at the best distance
#pragma unroll
        for (int j = 0; j < kPointQPL; ++j) {
            int found = -1;
            if (bg[j] >= 0) {
                for (int k = kPointGroup - 1; k >= 0; --k) {
                    const int pt = bg[j] + k;
                    if (pt < p1 && point_dist2<D>(x[j], dbase + (int64_t)pt * D) == bv[j]) found = pt;
                }
            }
            if (qp[j] < n && found >= 0)
                atomicMax(reinterpret_cast<unsigned long long*>(&keys[qp[j]]),
                          (unsigned long long)pack_key(-bv[j], (uint32_t)found));
        }
    }
}

__global__ void fill_u64_kernel(uint64_t* p, int64_t n, uint64_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ void fill_i32_kernel(int32_t* p, int64_t n, int32_t v) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

// Up to four fills in one launch (blockIdx.y selects the range; 4- or 8-byte elements).
struct FillRange { void* p; int64_t n; uint64_t v; int32_t bytes; };
struct FillSet { FillRange r[4]; };

__global__ void fill_multi_kernel(FillSet f) {
    const FillRange r = f.r[blockIdx.y];
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < r.n; i += (int64_t)gridDim.x * blockDim.x) {
        if (r.bytes == 8) static_cast<uint64_t*>(r.p)[i] = r.v;
        else static_cast<uint32_t*>(r.p)[i] = (uint32_t)r.v;
    }
}

// keys -> row ids for two key arrays in one launch (blockIdx.y selects), no scores
__global__ void decode_keys2_kernel(const uint64_t* k0, int64_t n0, int32_t* i0, const uint64_t* k1, int64_t n1,
                                    int32_t* i1) {
    const uint64_t* keys = blockIdx.y ? k1 : k0;
    int32_t* idx = blockIdx.y ? i1 : i0;
    const int64_t n = blockIdx.y ? n1 : n0;
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        idx[i] = key_row(keys[i]);
}

// keys -> row ids (and optionally scores; point searches store minus the squared
// distance, which `negate` turns back into the distance)
__global__ void decode_keys_kernel(const uint64_t* keys, int64_t n, int32_t* idx, float* score, int negate) {
    for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const uint64_t k = keys[i];
        idx[i] = key_row(k);
        if (score) {
            const float v = k ? from_ordered((uint32_t)(k >> 32)) : -INFINITY;
            score[i] = negate ? -v : v;
        }
    }
}

// Fast scheme set-up: per pixel of image a, state = -2 for seeds (live), -1 otherwise;
// seed k (row-major on the grid) goes to frontier slot k; counters and round-0 keys reset.
// Memo of the backward NN of the fast scheme: one int32 per pixel v of image 2 (per
// pair).  The NN of a pixel never changes, and a pixel of image 2 is often reached
// again in a later iteration (a chain that converges there lands on it twice), so each
// pixel's backward NN is searched once per call.  Rows and list entries are below 2^28.
constexpr int32_t kMemoRow = 0x0FFFFFFF;
constexpr int32_t kMemoFinal = 0x20000000;    // | u: NN(b[v], a) = u, found in an earlier iteration
constexpr int32_t kMemoPending = 0x40000000;  // | e: searched in this iteration, entry e of the list
constexpr int32_t kMemoClaimed = 0x7FFFFFFF;  // taken by this iteration's gather, entry not yet written
                                              // (0: never searched)

struct InitArgs {
    int32_t* state; int64_t n1; int32_t w;
    int32_t stride, offset, nx, nseeds;
    int32_t* front0; uint64_t* keys_f0; uint64_t* keys_b0; int64_t slot_stride;
    int32_t* cnt0; int32_t* cnt1;
    int32_t* memo; int64_t n2; int32_t* bcnt0; int32_t* bcnt1;
};

__global__ void fast_init_kernel(InitArgs a) {
    const int pair = blockIdx.y;
    const int64_t n = a.n1 > a.n2 ? a.n1 : a.n2;
    for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < n;
         p += (int64_t)gridDim.x * blockDim.x) {
        if (p < a.n1) {
            const int32_t y = (int32_t)(p / a.w), x = (int32_t)(p - (int64_t)y * a.w);
            const bool seed = y >= a.offset && x >= a.offset && (y - a.offset) % a.stride == 0 &&
                              (x - a.offset) % a.stride == 0;
            a.state[pair * a.n1 + p] = seed ? -2 : -1;
            if (seed) {
                const int64_t k = (int64_t)((y - a.offset) / a.stride) * a.nx + (x - a.offset) / a.stride;
                a.front0[pair * a.slot_stride + k] = (int32_t)p;
            }
        }
        if (p < a.nseeds) {
            a.keys_f0[pair * a.slot_stride + p] = 0;
            a.keys_b0[pair * a.slot_stride + p] = 0;
        }
        if (p < a.n2) a.memo[pair * a.n2 + p] = 0;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.cnt0[pair] = a.nseeds;
        a.cnt1[pair] = 0;
        a.bcnt0[pair] = 0;
        a.bcnt1[pair] = 0;
    }
}

// The backward queries of one iteration: the landing pixels v = NN(a[u], b) of the live
// pixels whose backward NN is not known yet, each once (a CAS on the memo claims v;
// ballot + prefix sum give each wave one atomic on the list count).  The list counts
// alternate between two per-pair counters: iteration t appends to bcnt and clears
// bcnt_next for iteration t + 1.
struct GatherArgs {
    const uint64_t* keys_f; const int32_t* cnt; int32_t* memo; int64_t n2;
    int32_t* blist; int32_t* bcnt; int32_t* bcnt_next; int64_t slot_stride;
};

__global__ __launch_bounds__(256) void fast_gather_kernel(GatherArgs a) {
    const int pair = blockIdx.y;
    const int n = a.cnt[pair];
    if (blockIdx.x == 0 && threadIdx.x == 0) a.bcnt_next[pair] = 0;
    const int lane = threadIdx.x & 63;
    int32_t* memo = a.memo + pair * a.n2;
    for (int64_t k0 = (int64_t)blockIdx.x * blockDim.x; k0 < n; k0 += (int64_t)gridDim.x * blockDim.x) {
        const int64_t k = k0 + threadIdx.x;
        int32_t v = -1;
        bool push = false;
        if (k < n) {
            v = key_row(a.keys_f[pair * a.slot_stride + k]);
            push = v >= 0 && v < a.n2 && memo[v] == 0 && atomicCAS(&memo[v], 0, kMemoClaimed) == 0;
        }
        const uint64_t mask = __ballot(push);
        if (mask) {
            const int leader = __ffsll((unsigned long long)mask) - 1;
            int at = 0;
            if (lane == leader) at = atomicAdd(&a.bcnt[pair], (int)__popcll(mask));
            at = __shfl(at, leader);
            if (push) {
                const int e = at + (int)__popcll(mask & __lanemask_lt());
                a.blist[pair * a.slot_stride + e] = v;
                memo[v] = kMemoPending | e;
            }
        }
    }
}

// One reciprocity check per live pixel u: v = NN(a[u], b), u' = NN(b[v], a), with u'
// from the memo (an earlier iteration) or from this iteration's backward keys (the
// memo's list entry; the first thread to read it records u' in the memo).
// u' == u: keep (u, v).  Otherwise u' becomes live next iteration if nobody has
// been there (state -1); ballot + prefix sum give each wave one atomic.
// The frontier counts rotate through three per-pair counters: iteration t reads
// cnt (its own count), adds the next frontier into cnt_next (cleared by iteration
// t - 1) and clears cnt_after for iteration t + 1; it also records its count in
// active[t].  The search kernels then only read their count.
struct CycleArgs {
    const int32_t* front; const uint64_t* keys_f; const uint64_t* keys_b;
    uint64_t* keys_f_next; uint64_t* keys_b_next; int32_t* front_next;
    const int32_t* cnt; int32_t* cnt_next; int32_t* cnt_after; int32_t* state;
    int32_t* active; int64_t active_stride;   // NULL, or this iteration's entry of [batch][max_iters]
    int64_t slot_stride; int64_t n1; int32_t last;
    int32_t* memo; int64_t n2;
};

__global__ __launch_bounds__(256) void fast_cycle_kernel(CycleArgs a) {
    const int pair = blockIdx.y;
    const int n = a.cnt[pair];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.cnt_after[pair] = 0;
        if (a.active) a.active[pair * a.active_stride] = n;
    }
    const int lane = threadIdx.x & 63;
    for (int k0 = blockIdx.x * blockDim.x; k0 < n; k0 += gridDim.x * blockDim.x) {
        const int k = k0 + threadIdx.x;
        bool push = false;
        int32_t u2 = -1;
        if (k < n) {
            const int64_t slot = pair * a.slot_stride + k;
            const int32_t u = a.front[slot];
            const int32_t v = key_row(a.keys_f[slot]);
            if (v >= 0 && v < a.n2) {
                int32_t* mv = a.memo + pair * a.n2 + v;
                const int32_t m = *mv;
                if (m & kMemoFinal) {
                    u2 = m & kMemoRow;
                } else if ((m & kMemoRow) < a.slot_stride) {
                    u2 = key_row(a.keys_b[pair * a.slot_stride + (m & kMemoRow)]);
                    if (u2 >= 0) *mv = kMemoFinal | u2;
                }
            }
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

// ---------------------------------------------------------------------------- matching loss

// The InfoNCE matching loss over ground-truth pairs M_gt of an image pair
// ("MASt3R dissection", section 3 "Napkin Formula"): pair (i, j) contributes
//     LSE_i - <a_i, b_j> / tau,   LSE_i = log sum_k exp(<a_i, b_k> / tau),
// the softmax running over every row k of map b.  lse_partial_kernel streams b
// against the rows i named by the ground truth with the similarity kernel's tiles
// and an online log-sum-exp epilogue (LseSum); nce_terms_kernel merges the
// partials of each pair in a fixed order and forms its term; nce_loss_kernel adds
// the terms of each image pair in a fixed order (in binary64).
struct NceArgs {
    const void* amap;        // [batch][n1][d] (image 1: the rows i)
    const void* bmap;        // [batch][n2][d] (image 2: the rows j and k)
    int64_t a_pair_elems;    // n1 * d
    int64_t b_pair_elems;    // n2 * d
    int32_t n1, n2, d;
    const int32_t* gt;       // [batch][n_gt][2] (i, j)
    int32_t n_gt;
    int32_t nseg;            // database segments, i.e. partials per ground-truth pair
    int32_t nblk;            // blocks of nce_terms_kernel per image pair
    float k2;                // log2(e) / tau
    float2* partial;         // [batch][n_gt][nseg] (m, s) of LseSum (base 2), merged over the lane halves
    float* terms;            // [batch][n_gt]
    float* lse2;             // NULL or [batch][n_gt]: the base-2 log-sum-exp of each pair
    double* block_sums;      // [batch][nblk]
    double* loss;            // [batch]
};

// Work item = (query group, database segment) as in nn_argmax_kernel, with the
// segment count fixed by the host so that partial[pair][t][segment] is written
// exactly once for every ground-truth pair t.  A ground-truth row out of range
// streams as a zero query (its term is set to NaN later).
template <int AR, int P>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(min_waves<AR, P>())))
void lse_partial_kernel(NceArgs a) {
    constexpr int QT = qt_of<AR, P>();
    constexpr int LDS_TILES = (AR == AR_BF16 ? 3 * kStageTiles : 2) * 32 * lds_row_bytes<AR, P>();
    __shared__ __attribute__((aligned(16))) char lds[LDS_TILES];
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.y;
    const int n = a.n_gt;
    const int ntiles = (a.n2 + 31) >> 5;
    const int nqt = (n + 31) >> 5;
    const int qgroups = (nqt + kWaves * QT - 1) / (kWaves * QT);
    const int nsg = a.nseg;
    const int items = qgroups * nsg;
    const void* qbase = pair_base<AR>(a.amap, a.a_pair_elems, pair);
    const char* dbytes = static_cast<const char*>(pair_base<AR>(a.bmap, a.b_pair_elems, pair));
    const int rb = row_bytes<AR>(a.d);
    const int32_t* gt = a.gt + (int64_t)pair * n * 2;

    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int qg = item / nsg;
        const int sg = item - qg * nsg;
        const int g0 = (int)((int64_t)qg * nqt / qgroups);
        const int g1 = (int)((int64_t)(qg + 1) * nqt / qgroups);
        const int nact = __builtin_amdgcn_readfirstlane(g0 + wv < g1 ? (g1 - g0 - wv + kWaves - 1) / kWaves : 0);
        Operand<AR, P> q[QT];
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            if (j < nact) {
                const int qp = (g0 + wv + j * kWaves) * 32 + jl;
                const int64_t row = qp < n ? gt[2 * qp] : -1;
                const bool valid = row >= 0 && row < a.n1;
                if constexpr (AR == AR_X3)
                    q[j].load_f32(static_cast<const float*>(qbase) + (valid ? row : 0) * a.d, valid, h, 1);
                else
                    q[j].load(qbase, valid ? row : 0, valid, h, a.d, 1);
            } else if constexpr (AR == AR_BF16) {
                q[j].load(qbase, 0, false, h, a.d, 1);   // zero: the register stream runs every slot
            }
        }
        const int t0 = (int)((int64_t)sg * ntiles / nsg);
        const int t1 = (int)((int64_t)(sg + 1) * ntiles / nsg);
        LseSum<QT> ep(a.k2);
        bool direct = false;
        if constexpr (AR == AR_BF16) direct = (int64_t)t1 * 32 <= a.n2;
        // bf16 segments without a ragged tile stream without LDS, each wave on its own
        // (empty query slots hold zero operands and are never written; a wave with no
        // query tile skips the stream); the choice is uniform over the workgroup, whose
        // staged path has barriers
        if (direct) {
            if constexpr (AR == AR_BF16)
                if (nact > 0) stream_regs<AR, P, 4>(dbytes, t0, t1, q, h, jl, a.d, ep);
        } else {
            stream_db<AR, P>(dbytes, rb, t0, t1, a.n2, lds, q, nact, h, jl, a.d, 2, ep);
        }
        // merge the two lane halves (disjoint rows of the same query)
#pragma unroll
        for (int j = 0; j < QT; ++j) {
            if (j < nact) {
                const float sj = ep.s[j] - ep.c[j];
                const float mo = __shfl_xor(ep.m[j], 32), so = __shfl_xor(sj, 32);
                const float m = __builtin_elementwise_maximum(ep.m[j], mo);
                // integer offsets: exact power-of-two scales (a half with m = -inf holds 0)
                const float s = (ep.m[j] == -INFINITY ? 0.0f : scale_pow2(sj, ep.m[j] - m)) +
                                (mo == -INFINITY ? 0.0f : scale_pow2(so, mo - m));
                const int qp = (g0 + wv + j * kWaves) * 32 + jl;
                if (h == 0 && qp < n) a.partial[((int64_t)pair * n + qp) * nsg + sg] = make_float2(m, s);
            }
        }
    }
}

__device__ __forceinline__ float elem_f32(float x) { return x; }
__device__ __forceinline__ float elem_f32(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }

// Per ground-truth pair t = (i, j), from the base-2 partials (m_seg, s_seg) (integer
// offsets m_seg): m = max m_seg, S = sum over segments (in order, compensated) of
// s_seg 2^(m_seg - m); S = S' 2^E with S' in [0.5, 1) and m' = m + E (exact), then
//     term = ln 2 * (m' - <a_i, b_j> * k2) + ln S',
// the positive score an fp32 dot product (components in order).  NaN when i or j is
// out of range.  Each block also leaves the binary64 sum of its terms.
template <typename T>
__global__ __launch_bounds__(256) void nce_terms_kernel(NceArgs a) {
    __shared__ double red[256];
    const int pair = blockIdx.y;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    double contrib = 0.0;
    if (t < a.n_gt) {
        const int64_t pt = (int64_t)pair * a.n_gt + t;
        const int i = a.gt[2 * pt], j = a.gt[2 * pt + 1];
        const float2* p = a.partial + pt * a.nseg;
        float m = -INFINITY;
        for (int k = 0; k < a.nseg; ++k) m = __builtin_elementwise_maximum(m, p[k].x);
        float S = 0.0f, c = 0.0f;
        for (int k = 0; k < a.nseg; ++k) {
            if (p[k].x == -INFINITY) continue;   // a segment with no row
            const float y = scale_pow2(p[k].y, p[k].x - m) - c;
            const float tot = S + y;
            c = (tot - S) - y;
            S = tot;
        }
        if (S > 0.0f && m != -INFINITY) {
            int e = 0;
            S = __builtin_frexpf(S, &e);
            m += (float)e;
        }
        if (a.lse2) a.lse2[pt] = m + log2f(S);
        float term = __builtin_nanf("");
        if (i >= 0 && i < a.n1 && j >= 0 && j < a.n2) {
            const T* x = static_cast<const T*>(a.amap) + pair * a.a_pair_elems + (int64_t)i * a.d;
            const T* y = static_cast<const T*>(a.bmap) + pair * a.b_pair_elems + (int64_t)j * a.d;
            float pos = 0.0f;
            for (int c = 0; c < a.d; ++c) pos = __builtin_fmaf(elem_f32(x[c]), elem_f32(y[c]), pos);
            term = 0.69314718055994531f * __builtin_fmaf(-pos, a.k2, m) + logf(S);
        }
        a.terms[pt] = term;
        contrib = term;
    }
    red[threadIdx.x] = contrib;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.block_sums[(int64_t)pair * a.nblk + blockIdx.x] = red[0];
}

// loss[pair] = sum of the pair's block sums (fixed order: strided, then a tree).
__global__ __launch_bounds__(256) void nce_loss_kernel(NceArgs a) {
    __shared__ double red[256];
    const int pair = blockIdx.x;
    double s = 0.0;
    for (int k = threadIdx.x; k < a.nblk; k += 256) s += a.block_sums[(int64_t)pair * a.nblk + k];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.loss[pair] = red[0];
}

// ---------------------------------------------------------------------------- matching loss, gradient

// With p[t][k] = 2^(<a_i, b_k> k2 - lse2_t) (term t's softmax over the rows k of b,
// lse2_t its base-2 log-sum-exp), the gradient of the summed loss is
//     dL/da_i = (1/tau) sum_{t: i_t = i} ( sum_k p[t][k] b_k - b_{j_t} ),
//     dL/db_k = (1/tau) sum_t p[t][k] a_{i_t} - (1/tau) sum_{t: j_t = k} a_{i_t}.
// Both softmax-weighted sums are attention-like products that nce_grad_kernel
// forms without storing p: the row pass takes the ground-truth rows a_{i_t} as
// queries and streams b (O_t = sum_k p[t][k] b_k); the column pass takes the rows
// of b as queries and streams the gathered rows a_{i_t} (O_k = sum_t p[t][k]
// a_{i_t}).  Per 32-row tile the scores come from the similarity MFMA (the same
// instruction, operand roles and order as the forward, so p is consistent with
// lse2), p from one fma and one v_exp per score, and O += p X on the matrix cores
// with p split into two bf16 parts (hi + lo, relative error below 2^-17) and X the
// staged tile read transposed (fp32 maps: its three bf16 planes).  d <= 32.
constexpr int kGradQT = 1;   // query tiles per wave
constexpr int kGradTStride = 36;   // halfwords per column of a transposed staged tile

struct NceGradArgs {
    const void* qmap;        // query rows: a (row pass, through the ground truth) or b (column pass)
    const void* xmap;        // streamed rows: b (row pass) or a (column pass, through the ground truth)
    int64_t q_pair_elems, x_pair_elems;
    int32_t nq_rows, nx_rows;  // rows of the query / streamed map per pair
    int32_t d;
    const int32_t* gt;       // [batch][n_gt][2]
    int32_t n_gt;
    int32_t nq, nx;          // queries and streamed rows per pair
    int32_t nseg;            // streamed segments (partials per query)
    float k2;                // log2(e) / tau
    const float* lse2;       // [batch][n_gt]
    float* partial;          // [batch][nq][nseg][32] fp32 (columns c < d used)
};

template <int AR, int P, bool COLS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(AR == AR_BF16 ? 4 : 2)))
void nce_grad_kernel(NceGradArgs a) {
    static_assert(AR == AR_BF16 || AR == AR_X3, "bf16 maps or the split fp32 arithmetic");
    using Elem = typename ArithTraits<AR>::elem;
    constexpr int TILE = 32 * lds_row_bytes<AR, P>();   // a staged 32-row tile: bf16 rows, or [h|m|l] planes
    constexpr int NPL = AR == AR_X3 ? 3 : 1;            // bf16 planes of a staged row
    // the same tile transposed, per plane: column c's 32 rows at c * kGradTStride
    // halfwords (8-byte aligned runs of 4 rows, padded against bank conflicts)
    constexpr int TILE_T = NPL * 32 * kGradTStride;      // halfwords
    __shared__ __attribute__((aligned(16))) char lds[2 * TILE];
    __shared__ __attribute__((aligned(16))) uint16_t ldsT[2 * TILE_T];
    __shared__ float lse_x[2][32];                    // column pass: lse2 of the staged rows
    const int lane = threadIdx.x & 63;
    const int h = lane >> 5;
    const int jl = lane & 31;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = blockIdx.y;
    const int d = a.d;
    const int rb = (int)sizeof(Elem) * d;             // bytes of a map row
    const int nq = a.nq, nx = a.nx, nsg = a.nseg;
    const int ntiles = (nx + 31) >> 5;
    const int nqt = (nq + 31) >> 5;
    const int qgroups = (nqt + kWaves * kGradQT - 1) / (kWaves * kGradQT);
    const int items = qgroups * nsg;
    const Elem* qbase = static_cast<const Elem*>(a.qmap) + pair * a.q_pair_elems;
    const char* xbytes = reinterpret_cast<const char*>(static_cast<const Elem*>(a.xmap) + pair * a.x_pair_elems);
    const int32_t* gt = a.gt + (int64_t)pair * a.n_gt * 2;
    const float* lse2 = a.lse2 + (int64_t)pair * a.n_gt;

    // row of the streamed map behind streamed index x (-1: none)
    auto x_row = [&](int x) -> int64_t {
        if (x >= nx) return -1;
        if (!COLS) return x;
        const int64_t r = gt[2 * x];
        return r >= 0 && r < a.nx_rows ? r : -1;
    };

    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int qg = item / nsg;
        const int sg = item - qg * nsg;
        const int g0 = (int)((int64_t)qg * nqt / qgroups);
        const int g1 = (int)((int64_t)(qg + 1) * nqt / qgroups);
        const int nact = __builtin_amdgcn_readfirstlane(g0 + wv < g1 ? (g1 - g0 - wv + kWaves - 1) / kWaves : 0);
        Operand<AR, P> q[kGradQT];
        float lq[kGradQT];                            // row pass: the query's lse2
#pragma unroll
        for (int j = 0; j < kGradQT; ++j) {
            lq[j] = INFINITY;
            if (j < nact) {
                const int qp = (g0 + wv + j * kWaves) * 32 + jl;
                int64_t row = -1;
                if (qp < nq) {
                    if (COLS) row = qp;
                    else {
                        row = gt[2 * qp];
                        lq[j] = lse2[qp];
                    }
                }
                const bool valid = row >= 0 && row < a.nq_rows;
                if constexpr (AR == AR_X3)
                    q[j].load_f32(reinterpret_cast<const float*>(qbase) + (valid ? row : 0) * d, valid, h, COLS ? 2 : 1);
                else
                    q[j].load(qbase, valid ? row : 0, valid, h, d, COLS ? 2 : 1);
            }
        }
        const int t0 = __builtin_amdgcn_readfirstlane((int)((int64_t)sg * ntiles / nsg));
        const int t1 = __builtin_amdgcn_readfirstlane((int)((int64_t)(sg + 1) * ntiles / nsg));
        f32x16 o[kGradQT];
#pragma unroll
        for (int j = 0; j < kGradQT; ++j) o[j] = f32x16{};

        // staging: 16-byte chunks of the tile's rows (zeros past the end), one per thread
        const int nchunk = 32 * rb / 16;
        auto fetch = [&](int t) {
            u32x4 v = {0u, 0u, 0u, 0u};
            if ((int)threadIdx.x < nchunk) {
                const int r = threadIdx.x / (rb / 16), cc = threadIdx.x - r * (rb / 16);
                const int64_t row = x_row(t * 32 + r);
                if (row >= 0) v = *reinterpret_cast<const u32x4*>(xbytes + row * rb + cc * 16);
            }
            return v;
        };
        auto fetch_lse = [&](int t) {
            const int x = t * 32 + (int)threadIdx.x;
            return COLS && threadIdx.x < 32 && x < nx ? lse2[x] : INFINITY;
        };
        auto put = [&](int buf, u32x4 v, float l) {
            if ((int)threadIdx.x < nchunk) {
                uint16_t* tdst = ldsT + buf * TILE_T;
                if constexpr (AR == AR_X3) {
                    // four fp32 components -> their h, m, l parts in the row's three planes
                    const int r = threadIdx.x / (d / 4), c0 = (threadIdx.x - r * (d / 4)) * 4;
                    uint2 e3[3];
                    split3x4(__uint_as_float(v[0]), __uint_as_float(v[1]), __uint_as_float(v[2]),
                             __uint_as_float(v[3]), e3);
                    char* dst = lds + buf * TILE + r * 6 * d + c0 * 2;
#pragma unroll
                    for (int k = 0; k < 3; ++k) {
                        *reinterpret_cast<uint2*>(dst + k * 2 * d) = e3[k];
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            tdst[(k * 32 + c0 + e) * kGradTStride + r] =
                                (uint16_t)((e & 1 ? (e < 2 ? e3[k].x : e3[k].y) >> 16 : (e < 2 ? e3[k].x : e3[k].y)) & 0xFFFF);
                    }
                } else {
                    *reinterpret_cast<u32x4*>(lds + buf * TILE + threadIdx.x * 16) = v;
                    const int r = threadIdx.x / (rb / 16), c0 = (threadIdx.x - r * (rb / 16)) * 8;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        tdst[(c0 + e) * kGradTStride + r] = (uint16_t)((v[e >> 1] >> (16 * (e & 1))) & 0xFFFF);
                }
            }
            if (COLS && threadIdx.x < 32) lse_x[buf][threadIdx.x] = l;
        };
        auto compute = [&](int buf, int t, auto ragged) {
            constexpr bool RAGGED = decltype(ragged)::value;
            const uint16_t* xs = reinterpret_cast<const uint16_t*>(lds + buf * TILE);
            Operand<AR, P> xo;
            if constexpr (AR == AR_BF16) {
                // k-slots past d repeat the row's first chunk: the query operand is zero
                // there, so the scores are unchanged (as in the search's register stream)
                int off[P];
                Operand<AR, P>::db_offsets(jl, h, d, off);
                xo.load_db(reinterpret_cast<const char*>(xs), off);
            } else {
                xo.load(xs, jl, true, h, d, COLS ? 1 : 2);
            }
            // the tile read transposed: lane (h, c) holds plane k of X[row R(s, h, e)][c],
            // e = 0..7, with R the accumulator's row order, so k-slot 8h + e of step s
            // pairs p and X.  R(s, h, e) runs over rows 16s + 4h + (0..3) for e < 4 and
            // 16s + 8 + 4h + (0..3) for e >= 4: two 8-byte reads of column c.
            bf16x8 xt[NPL][2];
            const uint16_t* xtc = ldsT + buf * TILE_T + (jl < d ? jl : 0) * kGradTStride + 4 * h;
#pragma unroll
            for (int k = 0; k < NPL; ++k)
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const uint2 lo4 = *reinterpret_cast<const uint2*>(xtc + k * 32 * kGradTStride + 16 * s2);
                    const uint2 hi4 = *reinterpret_cast<const uint2*>(xtc + k * 32 * kGradTStride + 16 * s2 + 8);
                    // (lanes c >= d repeat column 0: their output columns are never read)
                    const u32x4 w = {lo4.x, lo4.y, hi4.x, hi4.y};
                    xt[k][s2] = __builtin_bit_cast(bf16x8, w);
                }
            float lx[16];
            if (COLS) {
#pragma unroll
                for (int v = 0; v < 16; ++v) lx[v] = lse_x[buf][tile_row(v, h)];
            }
#pragma unroll
            for (int j = 0; j < kGradQT; ++j) {
                if (j < nact) {
                    const f32x16 acc = xo.mfma(q[j], f32x16{});
                    float pv[16];
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float lse = COLS ? lx[v] : lq[j];
                        pv[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[v], a.k2, -lse));
                        if (RAGGED && t * 32 + tile_row(v, h) >= nx) pv[v] = 0.0f;
                    }
                    // p = hi + lo, each rounded to bf16 in pairs (v_cvt_pk_bf16_f32)
                    bf16x8 ph[2], pl[2];
#pragma unroll
                    for (int v = 0; v < 16; v += 2) {
                        const bf16x2 hi = __builtin_convertvector(f32x2{pv[v], pv[v + 1]}, bf16x2);
                        const f32x2 back = __builtin_convertvector(hi, f32x2);
                        const bf16x2 lo = __builtin_convertvector(f32x2{pv[v] - back[0], pv[v + 1] - back[1]}, bf16x2);
                        ph[v >> 3][v & 7] = hi[0];
                        ph[v >> 3][(v & 7) + 1] = hi[1];
                        pl[v >> 3][v & 7] = lo[0];
                        pl[v >> 3][(v & 7) + 1] = lo[1];
                    }
#pragma unroll
                    for (int s2 = 0; s2 < 2; ++s2) {
                        // bf16 X: p_hi X + p_lo X.  Split X = X_h + X_m + X_l: the five
                        // products above 2^-24 of |p||X| (p_lo X_l is below it)
                        o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[s2], xt[0][s2], o[j], 0, 0, 0);
                        o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl[s2], xt[0][s2], o[j], 0, 0, 0);
                        if constexpr (NPL == 3) {
                            o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[s2], xt[1][s2], o[j], 0, 0, 0);
                            o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pl[s2], xt[1][s2], o[j], 0, 0, 0);
                            o[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ph[s2], xt[2][s2], o[j], 0, 0, 0);
                        }
                    }
                }
            }
        };

        if (t0 < t1) {
            // tile t + 1 is loaded into registers two iterations before it is written to
            // LDS (at the end of iteration t, after the multiply of tile t); loads past
            // the segment repeat its last tile, so they are issued unconditionally
            auto clamp = [&](int t) { return t < t1 ? t : t1 - 1; };
            u32x4 st[2];
            float sl[2];
            put(0, fetch(t0), fetch_lse(t0));
            st[0] = fetch(clamp(t0 + 1));
            sl[0] = fetch_lse(clamp(t0 + 1));
            st[1] = fetch(clamp(t0 + 2));
            sl[1] = fetch_lse(clamp(t0 + 2));
            __syncthreads();
            for (int t = t0; t < t1; t += 2) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int tt = t + u;
                    if (tt < t1) {
                        if ((tt + 1) * 32 > nx) compute(u, tt, std::true_type{});
                        else compute(u, tt, std::false_type{});
                        put(u ^ 1, st[u], sl[u]);
                        st[u] = fetch(clamp(tt + 3));
                        sl[u] = fetch_lse(clamp(tt + 3));
                        __syncthreads();
                    }
                }
            }
        }
        // lane (h, c) holds O[query tile_row(v, h)][c]
#pragma unroll
        for (int j = 0; j < kGradQT; ++j) {
            if (j < nact) {
                const int qb = (g0 + wv + j * kWaves) * 32;
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int qp = qb + tile_row(v, h);
                    if (qp < nq) a.partial[(((int64_t)pair * nq + qp) * nsg + sg) * 32 + jl] = o[j][v];
                }
            }
        }
    }
}

// Column pass result: db[k][c] = sum over segments (in order) of O_k[c], for every
// row k of b (binary64 scratch, written once).
__global__ __launch_bounds__(256) void nce_grad_cols_finish(NceGradArgs a, double* db) {
    const int pair = blockIdx.y;
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < (int64_t)a.nq * a.d; x += (int64_t)gridDim.x * 256) {
        const int64_t k = x / a.d;
        const int c = (int)(x - k * a.d);
        const float* p = a.partial + ((int64_t)pair * a.nq + k) * a.nseg * 32 + c;
        float s = 0.0f;
        for (int g = 0; g < a.nseg; ++g) s += p[g * 32];
        db[(int64_t)pair * a.nq * a.d + x] = (double)s;
    }
}

// Row pass result and the ground-truth terms of the gradient, per (t, c): da[i_t][c]
// += sum over segments of O_t[c] - b[j_t][c], and db[j_t][c] -= a[i_t][c] (binary64
// atomics; every addend is an fp32 value).  Pairs with an index out of range are
// skipped.
template <typename T>
__global__ __launch_bounds__(256) void nce_grad_rows_finish(NceGradArgs a, const T* amap, const T* bmap,
                                                            int64_t a_elems, int64_t b_elems, int32_t n1, int32_t n2,
                                                            double* da, double* db) {
    const int pair = blockIdx.y;
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < (int64_t)a.nq * a.d; x += (int64_t)gridDim.x * 256) {
        const int64_t t = x / a.d;
        const int c = (int)(x - t * a.d);
        const int32_t* g = a.gt + ((int64_t)pair * a.n_gt + t) * 2;
        const int i = g[0], j = g[1];
        if (i < 0 || i >= n1 || j < 0 || j >= n2) continue;
        const float* p = a.partial + ((int64_t)pair * a.nq + t) * a.nseg * 32 + c;
        float s = 0.0f;
        for (int k = 0; k < a.nseg; ++k) s += p[k * 32];
        double* dai = da + ((int64_t)pair * n1 + i) * a.d + c;
        double* dbj = db + ((int64_t)pair * n2 + j) * a.d + c;
        atomicAdd(dai, (double)s);
        atomicAdd(dai, -(double)elem_f32(bmap[pair * b_elems + (int64_t)j * a.d + c]));
        atomicAdd(dbj, -(double)elem_f32(amap[pair * a_elems + (int64_t)i * a.d + c]));
    }
}

// grad = acc / tau, rounded once to fp32.
__global__ __launch_bounds__(256) void nce_grad_scale(const double* acc, float* grad, int64_t n, double inv_tau) {
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256)
        grad[x] = (float)(acc[x] * inv_tau);
}

__global__ __launch_bounds__(256) void fill_f32_kernel(float* p, int64_t n, float v) {
    for (int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x; x < n; x += (int64_t)gridDim.x * 256) p[x] = v;
}

// ---------------------------------------------------------------------------- host helpers

// The measurement aid's window belongs to the thread that opened it: an entry point
// reads it only on that thread, so calls on other threads never touch it.  It holds
// no HIP object outside an open window (trivially destructible, no teardown work).
struct Profiler {
    bool on = false;
    int cap = 0, used = 0;
    hipEvent_t* ev = nullptr;
    int64_t* queries = nullptr;   // device [cap]: queries each timed search launch ran
    bool* counted = nullptr;      // host [cap]: whether the launch's entry of `queries` was written
};
thread_local Profiler g_prof;

// Queries a search launch runs, summed over the batch (its per-pair device counts, or
// the host count for every pair), into one entry of the profiling window.  Launched on
// the call's stream just before the launch's start event, so it is not timed.
__global__ __launch_bounds__(256) void prof_count_kernel(const int32_t* cnt, int64_t stride, int32_t host_n,
                                                         int32_t batch, int64_t* out) {
    __shared__ unsigned long long total;
    if (threadIdx.x == 0) total = 0;
    __syncthreads();
    unsigned long long part = 0;
    for (int p = threadIdx.x; p < batch; p += blockDim.x) part += (unsigned long long)(cnt ? cnt[p * stride] : host_n);
    atomicAdd(&total, part);
    __syncthreads();
    if (threadIdx.x == 0) *out = (int64_t)total;
}

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

// Workgroups for a grid-stride kernel over n items.  At most 2^20: the kernels loop
// over any n, and grid.x * threads must stay below the 2^32 work-items that one
// dimension of a dispatch can hold (2^24 workgroups of 256 would be exactly 2^32).
int grid_1d(int64_t n, int threads = 256, int cap = 1 << 20) {
    int64_t g = (n + threads - 1) / threads;
    if (g < 1) g = 1;
    return (int)(g > cap ? cap : g);
}

int dev_err() { return hipGetLastError() == hipSuccess ? MR_OK : MR_ERR_DEVICE; }

// hipEvents around one launch for the measurement aid (when it is on and has room).
int prof_mark(hipStream_t st, bool& rec) {
    rec = g_prof.on && g_prof.used < g_prof.cap;
    return rec && hipEventRecord(g_prof.ev[2 * g_prof.used], st) != hipSuccess ? MR_ERR_DEVICE : MR_OK;
}
int prof_close(hipStream_t st, bool rec) {
    if (!rec) return MR_OK;
    if (hipEventRecord(g_prof.ev[2 * g_prof.used + 1], st) != hipSuccess) return MR_ERR_DEVICE;
    ++g_prof.used;
    return MR_OK;
}


// Workgroups of kernel K (kThreads each) that the GPU holds at once: a launch-shape
// constant, computed once per process (a thread-safe static initialisation; a plain
// int, so process teardown has nothing to release).
template <auto K, int THREADS = kThreads>
int resident_blocks() {
    static const int resident = [] {
        int dev = 0, cus = 256, per_cu = 0;
        if (hipGetDevice(&dev) == hipSuccess) {
            hipDeviceProp_t prop;
            if (hipGetDeviceProperties(&prop, dev) == hipSuccess) cus = prop.multiProcessorCount;
        }
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, K, THREADS, 0) != hipSuccess || per_cu < 1)
            per_cu = 1;
        return cus * per_cu;
    }();
    return resident;
}

// Workgroups per pair: as many as the GPU holds at once (all pairs together); a
// multiple of 8 when large, so that work items keep to one XCD's share of the
// database rows.
inline int grid_per_pair(int resident, int batch) {
    int g = resident / (batch > 0 ? batch : 1);
    if (g >= 64) g &= ~7;
    return g < 1 ? 1 : g;
}

template <int AR, int P>
int nn_grid_x(int batch) {
    return grid_per_pair(resident_blocks<nn_argmax_kernel<AR, P>>(), batch);
}

// Workgroups are dealt to the eight XCDs round-robin by linear workgroup id, and each
// XCD has its own L2.  When a batch gives each pair only a few workgroups, a
// two-dimensional grid puts a pair's workgroups (its query groups) on different XCDs,
// and every XCD streams every pair's database map from memory.  For batches of a
// multiple of 8 pairs with 2..63 workgroups each, the grid is one-dimensional
// instead: linear id L runs pair (L mod 8) + 8 * ((L / 8) / gx), workgroup
// (L / 8) mod gx, so all of a pair's workgroups share the XCD L mod 8 and read its
// map through one L2.  Larger per-pair grids already keep one eighth of each map per
// XCD (segment counts are multiples of 8).
inline int xcd_packed_grid(int gx, int batch) {
    return (batch % 8 == 0 && gx > 1 && gx < 64) ? gx : 0;
}

template <int AR, int P>
void launch_nn_t(const NNArgs& a, int batch, hipStream_t st) {
    const int gx = nn_grid_x<AR, P>(batch);
    if (const int packed = xcd_packed_grid(gx, batch)) {
        NNArgs b = a;
        b.xcd_gx = packed;
        b.batch = batch;
        MR_LAUNCH((nn_argmax_kernel<AR, P>), dim3(packed * batch), dim3(kThreads), 0, st, b);
    } else {
        MR_LAUNCH((nn_argmax_kernel<AR, P>), dim3(gx, batch), dim3(kThreads), 0, st, a);
    }
}

// Arithmetic for a map dtype and descriptor length (see the Arith enum).
int choose_arith(int dtype, int d) {
    if (dtype == MR_BF16) return AR_BF16;
    return (d % 8 == 0 && d <= 32) ? AR_X3 : AR_F32;
}

// With a profiling window open: count the launch's queries, then its start event.
int prof_search_begin(const NNArgs& a, int batch, hipStream_t st, bool& prof) {
    prof = g_prof.on && g_prof.used < g_prof.cap;
    if (!prof) return MR_OK;
    MR_LAUNCH(prof_count_kernel, dim3(1), dim3(256), 0, st, a.dev_count, a.count_stride, a.host_count, batch,
              g_prof.queries + g_prof.used);
    if (dev_err()) return MR_ERR_DEVICE;
    g_prof.counted[g_prof.used] = true;
    return hipEventRecord(g_prof.ev[2 * g_prof.used], st) != hipSuccess ? MR_ERR_DEVICE : MR_OK;
}

int launch_nn(const NNArgs& a, int ar, int batch, hipStream_t st) {
    bool prof = false;
    if (prof_search_begin(a, batch, st, prof)) return MR_ERR_DEVICE;
    if (ar == AR_F32) {
        switch ((a.d + 1) / 2) {
#define MR_CASE(p) case p: launch_nn_t<AR_F32, p>(a, batch, st); break;
            MR_CASE(1) MR_CASE(2) MR_CASE(3) MR_CASE(4) MR_CASE(5) MR_CASE(6) MR_CASE(7) MR_CASE(8)
            MR_CASE(9) MR_CASE(10) MR_CASE(11) MR_CASE(12) MR_CASE(13) MR_CASE(14) MR_CASE(15) MR_CASE(16)
            MR_CASE(17) MR_CASE(18) MR_CASE(19) MR_CASE(20) MR_CASE(21) MR_CASE(22) MR_CASE(23) MR_CASE(24)
            MR_CASE(25) MR_CASE(26) MR_CASE(27) MR_CASE(28) MR_CASE(29) MR_CASE(30) MR_CASE(31) MR_CASE(32)
#undef MR_CASE
            default: return MR_ERR_SHAPE;
        }
    } else if (ar == AR_BF16) {
        switch ((a.d + 15) / 16) {
            case 1: launch_nn_t<AR_BF16, 1>(a, batch, st); break;
            case 2: launch_nn_t<AR_BF16, 2>(a, batch, st); break;
            case 3: launch_nn_t<AR_BF16, 3>(a, batch, st); break;
            case 4: launch_nn_t<AR_BF16, 4>(a, batch, st); break;
            default: return MR_ERR_SHAPE;
        }
    } else {
        switch (a.d) {
            case 8: launch_nn_t<AR_X3, 3>(a, batch, st); break;
            case 16: launch_nn_t<AR_X3, 6>(a, batch, st); break;
            case 24: launch_nn_t<AR_X3, 9>(a, batch, st); break;
            case 32: launch_nn_t<AR_X3, 12>(a, batch, st); break;
            default: return MR_ERR_SHAPE;
        }
    }
    if (dev_err()) return MR_ERR_DEVICE;
    if (prof) {
        if (hipEventRecord(g_prof.ev[2 * g_prof.used + 1], st) != hipSuccess) return MR_ERR_DEVICE;
        ++g_prof.used;
    }
    if (ar == AR_BF16) {
        // tile keys -> row keys
        const int64_t max_n = a.dev_count ? a.qlist_stride : a.host_count;
        const int gx = (int)((max_n + 31) / 32 < (1 << 20) ? (max_n + 31) / 32 : (1 << 20));
        if (gx < 1) return MR_OK;
        switch ((a.d + 15) / 16) {
#define MR_CASE(p) case p: MR_LAUNCH((recover_rows_kernel<AR_BF16, p>), dim3(gx, batch), dim3(kThreads), 0, st, a); break;
            MR_CASE(1) MR_CASE(2) MR_CASE(3) MR_CASE(4)
#undef MR_CASE
            default: return MR_ERR_SHAPE;
        }
        if (dev_err()) return MR_ERR_DEVICE;
    }
    return MR_OK;
}

// What "nearest" means for a call: the largest inner product (descriptor maps) or
// the smallest Euclidean distance (pointmaps).
enum Metric { M_INNER = 0, M_POINT = 1 };

template <int D>
void launch_point_t(const NNArgs& a, int batch, hipStream_t st) {
    const int g = grid_per_pair(resident_blocks<point_nn_kernel<D>>(), batch);
    MR_LAUNCH((point_nn_kernel<D>), dim3(g, batch), dim3(kThreads), 0, st, a);
}

// One NN search under a metric (the similarity kernel of every entry point).
int launch_search(const NNArgs& a, int metric, int ar, int batch, hipStream_t st) {
    if (metric != M_POINT) return launch_nn(a, ar, batch, st);
    bool prof = false;
    if (prof_search_begin(a, batch, st, prof)) return MR_ERR_DEVICE;
    switch (a.d) {
        case 1: launch_point_t<1>(a, batch, st); break;
        case 2: launch_point_t<2>(a, batch, st); break;
        case 3: launch_point_t<3>(a, batch, st); break;
        case 4: launch_point_t<4>(a, batch, st); break;
        default: return MR_ERR_SHAPE;
    }
    if (dev_err()) return MR_ERR_DEVICE;
    if (prof) {
        if (hipEventRecord(g_prof.ev[2 * g_prof.used + 1], st) != hipSuccess) return MR_ERR_DEVICE;
        ++g_prof.used;
    }
    return MR_OK;
}

// Maps valid for a metric: pointmaps are fp32 with at most 4 coordinates.
int validate_for(const mr_map* a, const mr_map* b, int metric) {
    const int rc = validate_pair(a, b);
    if (rc || metric != M_POINT) return rc;
    if (a->dtype != MR_F32) return MR_ERR_DTYPE;
    if (a->d > kMaxPointD) return MR_ERR_SHAPE;
    return MR_OK;
}

// Kernel arguments for queries taken from map q (role q_role) against map db.
NNArgs nn_args(const mr_map* q, const void* qdata, int q_role, const mr_map* db, const void* dbdata, int db_role) {
    NNArgs a;
    memset(&a, 0, sizeof(a));
    a.qmap = qdata;
    a.dbmap = dbdata;
    a.q_pair_elems = npix(q) * q->d;
    a.db_pair_elems = npix(db) * db->d;
    a.nq_rows = (int32_t)npix(q);
    a.ndb = (int32_t)npix(db);
    a.d = q->d;
    a.q_role = q_role;
    a.db_role = db_role;
    return a;
}

struct FastLayout {
    size_t keys_f[2], keys_b[2], front[2], cnt[3], state, blk, memo, blist, bcnt[2], total;
};

FastLayout fast_layout(const mr_map* a, const mr_map* b, int64_t nseeds) {
    FastLayout L;
    const int batch = a->batch;
    const int64_t n1 = npix(a);
    size_t off = 0;
    const size_t slots = (size_t)batch * (size_t)(nseeds > 0 ? nseeds : 1);
    for (int i = 0; i < 2; ++i) { L.keys_f[i] = off; off = align256(off + slots * 8); }
    for (int i = 0; i < 2; ++i) { L.keys_b[i] = off; off = align256(off + slots * 8); }
    for (int i = 0; i < 2; ++i) { L.front[i] = off; off = align256(off + slots * 4); }
    for (int i = 0; i < 3; ++i) { L.cnt[i] = off; off = align256(off + (size_t)batch * 4); }
    L.state = off; off = align256(off + (size_t)batch * (size_t)(n1 > 0 ? n1 : 1) * 4);
    L.blk = off; off = align256(off + (size_t)batch * (size_t)(nblk_of(n1) > 0 ? nblk_of(n1) : 1) * 4);
    const int64_t n2 = npix(b);
    L.memo = off; off = align256(off + (size_t)batch * (size_t)(n2 > 0 ? n2 : 1) * 4);
    L.blist = off; off = align256(off + slots * 4);
    for (int i = 0; i < 2; ++i) { L.bcnt[i] = off; off = align256(off + (size_t)batch * 4); }
    L.total = off;
    return L;
}

// Query blocks of the fused pass (kRcQT query tiles each) for a map of n pixels.
inline int64_t rc_blocks(int64_t n) { return ((n + 31) / 32 + kRcQT - 1) / kRcQT; }

struct MutualLayout { size_t keys_ab, keys_ba, blk, bcnt, bpos, blist, rcnt, rpos, rlist, total; };

MutualLayout mutual_layout(const mr_map* a, const mr_map* b) {
    MutualLayout L;
    const size_t batch = (size_t)a->batch;
    const int64_t na = npix(a), nb = npix(b);
    const size_t nbk = (size_t)(rc_blocks(na) > 0 ? rc_blocks(na) : 1);
    size_t off = 0;
    L.keys_ab = off; off = align256(off + batch * (size_t)(na > 0 ? na : 1) * 8);
    L.keys_ba = off; off = align256(off + batch * (size_t)(nb > 0 ? nb : 1) * 8);
    L.blk = off; off = align256(off + batch * (size_t)(nblk_of(na) > 0 ? nblk_of(na) : 1) * 4);
    // recoveries of the fused pass: per bucket counts, offsets and entries, for the
    // columns (b rows by winning query block) and the rows (queries by winning group of
    // kRcFlush b tiles)
    const size_t ntb = (size_t)(((nb + 31) / 32 + kRcFlush - 1) / kRcFlush > 0 ? ((nb + 31) / 32 + kRcFlush - 1) / kRcFlush : 1);
    L.bcnt = off; off = align256(off + batch * nbk * 4);
    L.bpos = off; off = align256(off + batch * nbk * 4);
    L.blist = off; off = align256(off + batch * (size_t)(nb > 0 ? nb : 1) * 4);
    L.rcnt = off; off = align256(off + batch * ntb * 4);
    L.rpos = off; off = align256(off + batch * ntb * 4);
    L.rlist = off; off = align256(off + batch * (size_t)(na > 0 ? na : 1) * 4);
    L.total = off;
    return L;
}

struct NNLayout { size_t keys, total; };

NNLayout nn_layout(const mr_map* q, const mr_map* db, int64_t n_q) {
    NNLayout L;
    size_t off = 0;
    L.keys = off; off = align256(off + (size_t)q->batch * (size_t)(n_q > 0 ? n_q : 1) * 8);
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

// A pair graph over a collection of maps: the collection with its batch replaced by
// the number of edges (the per-edge state is laid out like a batch of pairs), and
// the workspace bytes of the fast scheme over it plus the device copy of the edges.
mr_map graph_map(const mr_map* images, int32_t n_edges) {
    mr_map m = *images;
    m.batch = n_edges;
    return m;
}

size_t graph_edges_offset(const mr_map* g, int32_t stride, int32_t offset) {
    return fast_layout(g, g, seed_count(g->h, g->w, stride, offset)).total;
}

size_t graph_ws_bytes(const mr_map* images, int32_t n_edges, int32_t stride, int32_t offset) {
    const mr_map g = graph_map(images, n_edges);
    return align256(graph_edges_offset(&g, stride, offset) + (size_t)n_edges * 2 * sizeof(int32_t));
}

// The three calls, for either metric (the extern "C" entry points below name one).
int nn_impl(const mr_map* q, const mr_map* db, const int32_t* q_idx, int64_t n_q, int32_t* out_idx,
            float* out_score, void* ws, size_t ws_bytes, void* stream, int metric) {
    int rc = validate_for(q, db, metric);
    if (rc) return rc;
    if (n_q < 0 || n_q > (int64_t(1) << 28)) return MR_ERR_PARAM;
    if (!q_idx && n_q != npix(q)) return MR_ERR_PARAM;
    if (n_q == 0) return MR_OK;
    if (npix(q) == 0) return MR_ERR_SHAPE;  // query ids cannot name a row of an empty map
    if (!out_idx) return MR_ERR_NULL;
    const NNLayout L = nn_layout(q, db, n_q);
    if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    uint64_t* keys = at<uint64_t>(ws, L.keys);
    const int64_t tot = (int64_t)q->batch * n_q;
    MR_LAUNCH(fill_u64_kernel, dim3(grid_1d(tot)), dim3(256), 0, st, keys, tot, (uint64_t)0);
    if (dev_err()) return MR_ERR_DEVICE;
    NNArgs a = nn_args(q, q->data, 1, db, db->data, 2);
    a.qsrc = q_idx ? Q_LIST : Q_ALL;
    a.qlist = q_idx;
    a.qlist_stride = n_q;
    a.host_count = (int32_t)n_q;
    a.keys = keys;
    a.keys_stride = n_q;
    if ((rc = launch_search(a, metric, choose_arith(q->dtype, q->d), q->batch, st))) return rc;
    MR_LAUNCH(decode_keys_kernel, dim3(grid_1d(tot)), dim3(256), 0, st, keys, tot, out_idx, out_score,
                       (int)(metric == M_POINT));
    return dev_err();
}

// The fused row + column pass for bf16 maps (d <= 32): rowcol_argmax_kernel, then the
// two recoveries (tile -> row for the rows, query block -> row for the columns).  The
// keys are zero on entry.
template <int P>
int launch_rowcol_t(const mr_map* a, const mr_map* b, uint64_t* kab, uint64_t* kba, Buckets rb, Buckets cb,
                    hipStream_t st) {
    const int batch = a->batch;
    const int64_t na = npix(a), nb = npix(b);
    if (na == 0 || nb == 0) return MR_OK;
    RowColArgs x;
    memset(&x, 0, sizeof(x));
    x.amap = a->data;
    x.bmap = b->data;
    x.a_pair_elems = na * a->d;
    x.b_pair_elems = nb * b->d;
    x.na = (int32_t)na;
    x.nb = (int32_t)nb;
    x.d = a->d;
    x.keys_ab = kab;
    x.keys_ba = kba;
    // segments per query group: about three rounds of the resident workgroups, a
    // multiple of 8 when large (each XCD then streams the same eighth of b), at most
    // one per b tile
    const int resident = grid_per_pair(resident_blocks<rowcol_argmax_kernel<P>, kRcThreads>(), batch);
    const int64_t nqt = (na + 31) / 32, ntiles = (nb + 31) / 32;
    const int64_t qgroups = (nqt + kRcGroupTiles - 1) / kRcGroupTiles;
    int64_t nsg = (3 * (int64_t)resident + qgroups - 1) / qgroups;
    if (nsg >= 8) nsg = (nsg + 7) & ~int64_t(7);
    const int64_t ngroups = (ntiles + kRcFlush - 1) / kRcFlush;   // segments are whole groups
    const int64_t cap = ngroups < kMaxSegGroups ? ngroups : kMaxSegGroups;
    nsg = nsg < 1 ? 1 : (nsg > cap ? cap : nsg);
    x.nsg = (int32_t)nsg;
    const int64_t items = qgroups * nsg;
    const int gx = (int)(items < resident ? items : resident);
    bool rec = false;
    int rc;
    if ((rc = prof_mark(st, rec))) return rc;
    MR_LAUNCH((rowcol_argmax_kernel<P>), dim3(gx, batch), dim3(kRcThreads), 0, st, x);
    if (dev_err()) return MR_ERR_DEVICE;
    if ((rc = prof_close(st, rec))) return rc;
    // both directions' keys -> per-bucket lists (one launch per step for both; the
    // counts were zeroed with the keys), then one launch recovering both
    const int64_t nmax = rb.n > cb.n ? rb.n : cb.n;
    const int chunks = (int)((nmax + kBucketChunk - 1) / kBucketChunk);
    MR_LAUNCH(bucket_count_kernel, dim3(chunks, batch, 2), dim3(256), 0, st, rb, cb);
    MR_LAUNCH(bucket_scan_kernel, dim3(batch, 2), dim3(1024), 0, st, rb, cb);
    MR_LAUNCH(bucket_scatter_kernel, dim3(chunks, batch, 2), dim3(256), 0, st, rb, cb);
    const int nbmax = rb.nbins > cb.nbins ? rb.nbins : cb.nbins;
    MR_LAUNCH((recover_rowcol_kernel<P>), dim3(nbmax < 65536 ? nbmax : 65536, batch, 2), dim3(kThreads), 0, st,
                       x, rb, cb);
    return dev_err();
}

int launch_rowcol(const mr_map* a, const mr_map* b, uint64_t* kab, uint64_t* kba, Buckets rb, Buckets cb,
                  hipStream_t st) {
    switch ((a->d + 15) / 16) {
        case 1: return launch_rowcol_t<1>(a, b, kab, kba, rb, cb, st);
        case 2: return launch_rowcol_t<2>(a, b, kab, kba, rb, cb, st);
        default: return MR_ERR_SHAPE;
    }
}

int mutual_impl(const mr_map* a, const mr_map* b, int32_t* nn_ab, int32_t* nn_ba, int32_t* pairs, int64_t cap,
                int64_t* n_pairs, void* ws, size_t ws_bytes, void* stream, int metric) {
    int rc = validate_for(a, b, metric);
    if (rc) return rc;
    if (!nn_ab || !nn_ba || !pairs || !n_pairs) return MR_ERR_NULL;
    const int64_t na = npix(a), nb = npix(b);
    const int64_t bound = na < nb ? na : nb;
    if (cap < bound) return MR_ERR_CAPACITY;
    const MutualLayout L = mutual_layout(a, b);
    if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int batch = a->batch;
    const int ar = choose_arith(a->dtype, a->d);
    uint64_t* kab = at<uint64_t>(ws, L.keys_ab);
    uint64_t* kba = at<uint64_t>(ws, L.keys_ba);
    int32_t* blk = at<int32_t>(ws, L.blk);
    const bool fused = metric == M_INNER && ar == AR_BF16 && a->d <= 32;
    Buckets rb{kab, na, at<int32_t>(ws, L.rcnt), at<int32_t>(ws, L.rpos), at<int32_t>(ws, L.rlist),
               (int32_t)(((nb + 31) / 32 + kRcFlush - 1) / kRcFlush)};
    Buckets cb{kba, nb, at<int32_t>(ws, L.bcnt), at<int32_t>(ws, L.bpos), at<int32_t>(ws, L.blist),
               (int32_t)rc_blocks(na)};
    // zero the keys (and the fused pass's bucket counts) in one launch
    FillSet fs;
    memset(&fs, 0, sizeof(fs));
    fs.r[0] = FillRange{kab, batch * na, 0, 8};
    fs.r[1] = FillRange{kba, batch * nb, 0, 8};
    if (fused) {
        fs.r[2] = FillRange{rb.cnt, batch * (int64_t)rb.nbins, 0, 4};
        fs.r[3] = FillRange{cb.cnt, batch * (int64_t)cb.nbins, 0, 4};
    }
    MR_LAUNCH(fill_multi_kernel, dim3(grid_1d(batch * (na > nb ? na : nb)), fused ? 4 : 2), dim3(256), 0, st,
                       fs);
    if (dev_err()) return MR_ERR_DEVICE;
    const void *ad = a->data, *bd = b->data;
    if (fused) {
        // both directions from one pass over the similarity tiles
        if ((rc = launch_rowcol(a, b, kab, kba, rb, cb, st))) return rc;
    } else {
        NNArgs f = nn_args(a, ad, 1, b, bd, 2);
        f.qsrc = Q_ALL;
        f.host_count = (int32_t)na;
        f.keys = kab;
        f.keys_stride = na;
        if ((rc = launch_search(f, metric, ar, batch, st))) return rc;
        NNArgs r = nn_args(b, bd, 2, a, ad, 1);
        r.qsrc = Q_ALL;
        r.host_count = (int32_t)nb;
        r.keys = kba;
        r.keys_stride = nb;
        if ((rc = launch_search(r, metric, ar, batch, st))) return rc;
    }
    MR_LAUNCH(decode_keys2_kernel, dim3(grid_1d(batch * (na > nb ? na : nb)), 2), dim3(256), 0, st, kab,
                       batch * na, nn_ab, kba, batch * nb, nn_ba);
    if (dev_err()) return MR_ERR_DEVICE;
    const int nblk = nblk_of(na) > 0 ? nblk_of(na) : 1;
    MutualPred pr{nn_ab, nn_ba, na, nb};
    MR_LAUNCH(compact_count_kernel<MutualPred>, dim3(nblk, batch), dim3(256), 0, st, pr, na, blk, nblk);
    MR_LAUNCH(compact_scatter_kernel<MutualPred>, dim3(nblk, batch), dim3(256), 0, st, pr, na,
                       (const int32_t*)blk, nblk, pairs, cap, n_pairs);
    return dev_err();
}

// edges: NULL, or the device edge table of a pair graph ([batch][2] map ids into a and
// b, which then hold the whole collection at their base while their batch counts the
// edges); the caller has validated it and its workspace region.
int fast_impl(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset, int32_t max_iters, int32_t* pairs,
              int64_t cap, int64_t* n_pairs, int32_t* iter_active, void* ws, size_t ws_bytes, void* stream,
              int metric, const int32_t* edges = nullptr) {
    int rc = validate_for(a, b, metric);
    if (rc) return rc;
    if (stride < 1 || offset < 0 || max_iters < 0) return MR_ERR_PARAM;
    if (!pairs || !n_pairs) return MR_ERR_NULL;
    const int64_t ns = seed_count(a->h, a->w, stride, offset);
    if (cap < ns) return MR_ERR_CAPACITY;
    const int64_t n1 = npix(a), n2 = npix(b);
    const FastLayout L = fast_layout(a, b, ns);
    if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int batch = a->batch;
    const int ar = choose_arith(a->dtype, a->d);
    const int64_t slot = ns > 0 ? ns : 1;
    uint64_t* kf[2] = {at<uint64_t>(ws, L.keys_f[0]), at<uint64_t>(ws, L.keys_f[1])};
    uint64_t* kb[2] = {at<uint64_t>(ws, L.keys_b[0]), at<uint64_t>(ws, L.keys_b[1])};
    int32_t* fr[2] = {at<int32_t>(ws, L.front[0]), at<int32_t>(ws, L.front[1])};
    int32_t* cnt[3] = {at<int32_t>(ws, L.cnt[0]), at<int32_t>(ws, L.cnt[1]), at<int32_t>(ws, L.cnt[2])};
    int32_t* state = at<int32_t>(ws, L.state);
    int32_t* blk = at<int32_t>(ws, L.blk);
    int32_t* memo = at<int32_t>(ws, L.memo);
    int32_t* blist = at<int32_t>(ws, L.blist);
    int32_t* bcnt[2] = {at<int32_t>(ws, L.bcnt[0]), at<int32_t>(ws, L.bcnt[1])};

    InitArgs ia;
    ia.state = state; ia.n1 = n1; ia.w = a->w; ia.stride = stride; ia.offset = offset;
    ia.nx = (int32_t)(offset < a->w ? (a->w - 1 - offset) / stride + 1 : 0);
    ia.nseeds = (int32_t)ns;
    ia.front0 = fr[0]; ia.keys_f0 = kf[0]; ia.keys_b0 = kb[0]; ia.slot_stride = slot;
    ia.cnt0 = cnt[0]; ia.cnt1 = cnt[1];
    ia.memo = memo; ia.n2 = n2; ia.bcnt0 = bcnt[0]; ia.bcnt1 = bcnt[1];
    const int64_t init_n = n1 > n2 ? n1 : n2;
    MR_LAUNCH(fast_init_kernel, dim3(grid_1d(init_n > 0 ? init_n : 1), batch), dim3(256), 0, st, ia);
    if (dev_err()) return MR_ERR_DEVICE;

    if (n1 > 0 && n2 > 0 && ns > 0 && max_iters > 0) {
        const void *ad = a->data, *bd = b->data;
        const int cyc_grid = grid_1d(ns);
        for (int t = 0; t < max_iters; ++t) {
            const int c = t & 1, x = c ^ 1;
            NNArgs f = nn_args(a, ad, 1, b, bd, 2);
            if (edges) { f.q_img = edges; f.db_img = edges + 1; }
            f.qsrc = Q_LIST; f.qlist = fr[c]; f.qlist_stride = slot;
            f.dev_count = cnt[t % 3]; f.count_stride = 1;
            f.keys = kf[c]; f.keys_stride = slot;
            if ((rc = launch_search(f, metric, ar, batch, st))) return rc;
            GatherArgs ga;
            ga.keys_f = kf[c]; ga.cnt = cnt[t % 3]; ga.memo = memo; ga.n2 = n2;
            ga.blist = blist; ga.bcnt = bcnt[c]; ga.bcnt_next = bcnt[x]; ga.slot_stride = slot;
            MR_LAUNCH(fast_gather_kernel, dim3(cyc_grid, batch), dim3(256), 0, st, ga);
            if (dev_err()) return MR_ERR_DEVICE;
            NNArgs r = nn_args(b, bd, 2, a, ad, 1);
            if (edges) { r.q_img = edges + 1; r.db_img = edges; }
            r.qsrc = Q_LIST; r.qlist = blist; r.qlist_stride = slot;
            r.dev_count = bcnt[c]; r.count_stride = 1;
            r.keys = kb[c]; r.keys_stride = slot;
            if ((rc = launch_search(r, metric, ar, batch, st))) return rc;
            CycleArgs ca;
            ca.front = fr[c]; ca.keys_f = kf[c]; ca.keys_b = kb[c];
            ca.keys_f_next = kf[x]; ca.keys_b_next = kb[x]; ca.front_next = fr[x];
            ca.cnt = cnt[t % 3]; ca.cnt_next = cnt[(t + 1) % 3]; ca.cnt_after = cnt[(t + 2) % 3];
            ca.state = state;
            ca.active = iter_active ? iter_active + t : nullptr; ca.active_stride = max_iters;
            ca.slot_stride = slot; ca.n1 = n1; ca.last = (t == max_iters - 1);
            ca.memo = memo; ca.n2 = n2;
            MR_LAUNCH(fast_cycle_kernel, dim3(cyc_grid, batch), dim3(256), 0, st, ca);
            if (dev_err()) return MR_ERR_DEVICE;
        }
    } else if (iter_active && max_iters > 0) {
        // nothing to search: every iteration has no live pixel
        const int64_t n = (int64_t)batch * max_iters;
        MR_LAUNCH(fill_i32_kernel, dim3(grid_1d(n)), dim3(256), 0, st, iter_active, n, 0);
        if (dev_err()) return MR_ERR_DEVICE;
    }
    const int nblk = nblk_of(n1) > 0 ? nblk_of(n1) : 1;
    FastPred pr{state, n1};
    MR_LAUNCH(compact_count_kernel<FastPred>, dim3(nblk, batch), dim3(256), 0, st, pr, n1, blk, nblk);
    MR_LAUNCH(compact_scatter_kernel<FastPred>, dim3(nblk, batch), dim3(256), 0, st, pr, n1,
                       (const int32_t*)blk, nblk, pairs, cap, n_pairs);
    return dev_err();
}


// ---------------------------------------------------------------------------- matching loss (host)

// The kernel instance for a map dtype and d: bf16 maps on the bf16 products, fp32
// maps on the exact three-way split (d a multiple of 8, at most 32).  f receives
// the arithmetic and the step count as integral constants.
template <class F>
int with_lse_arith(int dtype, int d, F&& f) {
    using std::integral_constant;
    if (dtype == MR_BF16) {
        switch ((d + 15) / 16) {
            case 1: return f(integral_constant<int, AR_BF16>{}, integral_constant<int, 1>{});
            case 2: return f(integral_constant<int, AR_BF16>{}, integral_constant<int, 2>{});
            case 3: return f(integral_constant<int, AR_BF16>{}, integral_constant<int, 3>{});
            case 4: return f(integral_constant<int, AR_BF16>{}, integral_constant<int, 4>{});
            default: return MR_ERR_SHAPE;
        }
    }
    switch (d) {
        case 8: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 3>{});
        case 16: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 6>{});
        case 24: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 9>{});
        case 32: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 12>{});
        default: return MR_ERR_SHAPE;
    }
}

struct NceLayout {
    int grid = 0, nseg = 0, nblk = 0;
    size_t partial = 0, sums = 0, total = 0;
};

// Launch shape and workspace of the matching loss: segments per query group as
// for the NN search (the resident workgroups spread over the query groups, a
// multiple of 8 when large, at most one per database tile).
int nce_layout(const mr_map* a, const mr_map* b, int64_t n_gt, NceLayout& L) {
    return with_lse_arith(a->dtype, a->d, [&](auto ar, auto p) {
        constexpr int AR = decltype(ar)::value, P = decltype(p)::value;
        constexpr int QT = qt_of<AR, P>();
        const int g = grid_per_pair(resident_blocks<lse_partial_kernel<AR, P>>(), a->batch);
        const int64_t ntiles = (npix(b) + 31) / 32;
        const int64_t qgroups = ((n_gt + 31) / 32 + kWaves * QT - 1) / (kWaves * QT);
        int64_t nseg = qgroups > 0 ? g / qgroups : 1;
        const int64_t cap = ntiles < kMaxSegGroups ? ntiles : kMaxSegGroups;
        nseg = nseg < 1 ? 1 : (nseg > cap ? cap : nseg);
        if (nseg >= 8) nseg &= ~int64_t(7);
        L.nseg = (int)nseg;
        L.grid = (int)(qgroups * nseg < g ? qgroups * nseg : g);
        L.nblk = (int)((n_gt + 255) / 256);
        size_t off = 0;
        const size_t rows = (size_t)a->batch * (size_t)(n_gt > 0 ? n_gt : 1);
        L.partial = off; off = align256(off + rows * (size_t)nseg * sizeof(float2));
        L.sums = off; off = align256(off + (size_t)a->batch * (size_t)(L.nblk > 0 ? L.nblk : 1) * sizeof(double));
        L.total = off;
        return (int)MR_OK;
    });
}

int validate_nce(const mr_map* a, const mr_map* b, int64_t n_gt) {
    const int rc = validate_pair(a, b);
    if (rc) return rc;
    if (n_gt < 0 || n_gt > (int64_t(1) << 28)) return MR_ERR_PARAM;
    if (npix(b) == 0) return MR_ERR_SHAPE;   // the softmax needs at least one row
    if (n_gt > 0 && npix(a) == 0) return MR_ERR_SHAPE;   // no ground-truth row can name a row of an empty map
    if (a->dtype == MR_F32 && (a->d % 8 != 0 || a->d > 32)) return MR_ERR_SHAPE;
    return MR_OK;
}

// The forward stages: log-sum-exp partials, terms (and lse2 when asked), loss.
// Arguments are validated and n_gt > 0.
int nce_forward_launch(const mr_map* a, const mr_map* b, const int32_t* gt, int64_t n_gt, float tau,
                       const NceLayout& L, void* ws, float* out_terms, double* out_loss, float* lse2, bool timed,
                       hipStream_t st) {
    const int batch = a->batch;
    NceArgs x;
    memset(&x, 0, sizeof(x));
    x.amap = a->data;
    x.bmap = b->data;
    x.a_pair_elems = npix(a) * a->d;
    x.b_pair_elems = npix(b) * b->d;
    x.n1 = (int32_t)npix(a);
    x.n2 = (int32_t)npix(b);
    x.d = a->d;
    x.gt = gt;
    x.n_gt = (int32_t)n_gt;
    x.nseg = L.nseg;
    x.nblk = L.nblk;
    x.k2 = (float)(1.4426950408889634 / (double)tau);
    x.partial = at<float2>(ws, L.partial);
    x.terms = out_terms;
    x.lse2 = lse2;
    x.block_sums = at<double>(ws, L.sums);
    x.loss = out_loss;
    bool rec = false;
    int rc;
    if (timed && (rc = prof_mark(st, rec))) return rc;
    rc = with_lse_arith(a->dtype, a->d, [&](auto ar, auto p) {
        constexpr int AR = decltype(ar)::value, P = decltype(p)::value;
        MR_LAUNCH((lse_partial_kernel<AR, P>), dim3(L.grid, batch), dim3(kThreads), 0, st, x);
        return dev_err();
    });
    if (rc || (rc = prof_close(st, rec))) return rc;
    if (a->dtype == MR_BF16)
        MR_LAUNCH(nce_terms_kernel<uint16_t>, dim3(L.nblk, batch), dim3(256), 0, st, x);
    else
        MR_LAUNCH(nce_terms_kernel<float>, dim3(L.nblk, batch), dim3(256), 0, st, x);
    if (dev_err()) return MR_ERR_DEVICE;
    MR_LAUNCH(nce_loss_kernel, dim3(batch), dim3(256), 0, st, x);
    return dev_err();
}

int fill_zero(void* p, int64_t words, hipStream_t st) {   // words of 8 bytes
    if (words <= 0) return MR_OK;
    MR_LAUNCH(fill_u64_kernel, dim3(grid_1d(words)), dim3(256), 0, st, static_cast<uint64_t*>(p), words,
                       (uint64_t)0);
    return dev_err();
}

int infonce_impl(const mr_map* a, const mr_map* b, const int32_t* gt, int64_t n_gt, float tau, float* out_terms,
                 double* out_loss, void* ws, size_t ws_bytes, void* stream) {
    int rc = validate_nce(a, b, n_gt);
    if (rc) return rc;
    if (!(tau > 0.0f) || !(tau < INFINITY)) return MR_ERR_PARAM;
    if (!out_loss) return MR_ERR_NULL;
    if (n_gt > 0 && (!gt || !out_terms)) return MR_ERR_NULL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (n_gt == 0) return fill_zero(out_loss, a->batch, st);   // +0.0
    NceLayout L;
    if ((rc = nce_layout(a, b, n_gt, L))) return rc;
    if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
    return nce_forward_launch(a, b, gt, n_gt, tau, L, ws, out_terms, out_loss, nullptr, true, st);
}

// ---- gradient

struct NceGradLayout {
    NceLayout f;
    int nseg_r = 0, nseg_c = 0, grid_r = 0, grid_c = 0;
    size_t lse2 = 0, prow = 0, pcol = 0, da = 0, db = 0, total = 0;
};

// Segments of a gradient pass as for the forward: resident workgroups spread over the
// query groups, at most one per streamed tile, a multiple of 8 when large.
template <int AR, int P, bool COLS>
void grad_pass_shape(int batch, int64_t nq, int64_t nx, int& nseg, int& grid) {
    const int g = grid_per_pair(resident_blocks<nce_grad_kernel<AR, P, COLS>>(), batch);
    const int64_t ntiles = (nx + 31) / 32;
    const int64_t qgroups = ((nq + 31) / 32 + kWaves * kGradQT - 1) / (kWaves * kGradQT);
    int64_t ns = qgroups > 0 ? g / qgroups : 1;
    const int64_t cap = ntiles < kMaxSegGroups ? ntiles : kMaxSegGroups;
    ns = ns < 1 ? 1 : (ns > cap ? cap : ns);
    if (ns >= 8) ns &= ~int64_t(7);
    nseg = (int)ns;
    grid = (int)(qgroups * ns < g ? qgroups * ns : g);
    if (grid < 1) grid = 1;
}

int validate_nce_grad(const mr_map* a, const mr_map* b, int64_t n_gt) {
    const int rc = validate_nce(a, b, n_gt);
    if (rc) return rc;
    if (a->d > 32) return MR_ERR_SHAPE;   // fp32 maps are already held to d in {8, 16, 24, 32}
    return MR_OK;
}

// The gradient kernel instance for a map dtype and d (bf16: P = ceil(d / 16) steps;
// fp32: the split arithmetic, P = 3d / 8), as integral constants to f.
template <class F>
int with_grad_arith(int dtype, int d, F&& f) {
    using std::integral_constant;
    if (dtype == MR_BF16) {
        if (d <= 16) return f(integral_constant<int, AR_BF16>{}, integral_constant<int, 1>{});
        if (d <= 32) return f(integral_constant<int, AR_BF16>{}, integral_constant<int, 2>{});
        return MR_ERR_SHAPE;
    }
    switch (d) {
        case 8: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 3>{});
        case 16: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 6>{});
        case 24: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 9>{});
        case 32: return f(integral_constant<int, AR_X3>{}, integral_constant<int, 12>{});
        default: return MR_ERR_SHAPE;
    }
}

int nce_grad_layout(const mr_map* a, const mr_map* b, int64_t n_gt, NceGradLayout& L) {
    const int rc = nce_layout(a, b, n_gt, L.f);
    if (rc) return rc;
    const int64_t n1 = npix(a), n2 = npix(b);
    const int batch = a->batch;
    const int rs = with_grad_arith(a->dtype, a->d, [&](auto ar, auto p) {
        constexpr int AR = decltype(ar)::value, P = decltype(p)::value;
        grad_pass_shape<AR, P, false>(batch, n_gt, n2, L.nseg_r, L.grid_r);
        grad_pass_shape<AR, P, true>(batch, n2, n_gt, L.nseg_c, L.grid_c);
        return (int)MR_OK;
    });
    if (rs) return rs;
    const size_t B = (size_t)batch, d = (size_t)a->d, ngt = (size_t)(n_gt > 0 ? n_gt : 1);
    size_t off = L.f.total;
    L.lse2 = off; off = align256(off + B * ngt * sizeof(float));
    L.prow = off; off = align256(off + B * ngt * (size_t)L.nseg_r * 32 * sizeof(float));
    L.pcol = off; off = align256(off + B * (size_t)n2 * (size_t)L.nseg_c * 32 * sizeof(float));
    L.da = off; off = align256(off + B * (size_t)(n1 > 0 ? n1 : 1) * d * sizeof(double));
    L.db = off; off = align256(off + B * (size_t)n2 * d * sizeof(double));
    L.total = off;
    return MR_OK;
}

int infonce_backward_impl(const mr_map* a, const mr_map* b, const int32_t* gt, int64_t n_gt, float tau,
                          float* out_terms, double* out_loss, float* grad_a, float* grad_b, void* ws,
                          size_t ws_bytes, void* stream) {
    int rc = validate_nce_grad(a, b, n_gt);
    if (rc) return rc;
    if (!(tau > 0.0f) || !(tau < INFINITY)) return MR_ERR_PARAM;
    const int64_t n1 = npix(a), n2 = npix(b);
    if (!out_loss || !grad_b || (n1 > 0 && !grad_a)) return MR_ERR_NULL;
    if (n_gt > 0 && (!gt || !out_terms)) return MR_ERR_NULL;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int batch = a->batch;
    const int d = a->d;
    if (n_gt == 0) {   // loss 0, gradients 0
        if ((rc = fill_zero(out_loss, batch, st))) return rc;
        if (n1 > 0)
            MR_LAUNCH(fill_f32_kernel, dim3(grid_1d(batch * n1 * d)), dim3(256), 0, st, grad_a,
                               (int64_t)batch * n1 * d, 0.0f);
        MR_LAUNCH(fill_f32_kernel, dim3(grid_1d(batch * n2 * d)), dim3(256), 0, st, grad_b,
                           (int64_t)batch * n2 * d, 0.0f);
        return dev_err();
    }
    NceGradLayout L;
    if ((rc = nce_grad_layout(a, b, n_gt, L))) return rc;
    if ((rc = check_ws(ws, ws_bytes, L.total))) return rc;
    double* da = at<double>(ws, L.da);
    double* db = at<double>(ws, L.db);
    float* lse2 = at<float>(ws, L.lse2);
    if ((rc = fill_zero(da, (int64_t)batch * n1 * d, st))) return rc;
    if ((rc = nce_forward_launch(a, b, gt, n_gt, tau, L.f, ws, out_terms, out_loss, lse2, false, st))) return rc;

    NceGradArgs r;
    memset(&r, 0, sizeof(r));
    r.d = d;
    r.gt = gt;
    r.n_gt = (int32_t)n_gt;
    r.k2 = (float)(1.4426950408889634 / (double)tau);
    r.lse2 = lse2;
    NceGradArgs c = r;
    r.qmap = a->data; r.xmap = b->data; r.q_pair_elems = n1 * d; r.x_pair_elems = n2 * d;
    r.nq_rows = (int32_t)n1; r.nx_rows = (int32_t)n2; r.nq = (int32_t)n_gt; r.nx = (int32_t)n2;
    r.nseg = L.nseg_r; r.partial = at<float>(ws, L.prow);
    c.qmap = b->data; c.xmap = a->data; c.q_pair_elems = n2 * d; c.x_pair_elems = n1 * d;
    c.nq_rows = (int32_t)n2; c.nx_rows = (int32_t)n1; c.nq = (int32_t)n2; c.nx = (int32_t)n_gt;
    c.nseg = L.nseg_c; c.partial = at<float>(ws, L.pcol);
    rc = with_grad_arith(a->dtype, d, [&](auto ar, auto p) {
        constexpr int AR = decltype(ar)::value, P = decltype(p)::value;
        bool rec = false;
        int e;
        if ((e = prof_mark(st, rec))) return e;
        MR_LAUNCH((nce_grad_kernel<AR, P, false>), dim3(L.grid_r, batch), dim3(kThreads), 0, st, r);
        if (dev_err()) return (int)MR_ERR_DEVICE;
        if ((e = prof_close(st, rec)) || (e = prof_mark(st, rec))) return e;
        MR_LAUNCH((nce_grad_kernel<AR, P, true>), dim3(L.grid_c, batch), dim3(kThreads), 0, st, c);
        if (dev_err()) return (int)MR_ERR_DEVICE;
        return prof_close(st, rec);
    });
    if (rc) return rc;
    MR_LAUNCH(nce_grad_cols_finish, dim3(grid_1d(n2 * d), batch), dim3(256), 0, st, c, db);
    if (dev_err()) return MR_ERR_DEVICE;
    if (a->dtype == MR_BF16)
        MR_LAUNCH(nce_grad_rows_finish<uint16_t>, dim3(grid_1d(n_gt * d), batch), dim3(256), 0, st, r,
                           static_cast<const uint16_t*>(a->data), static_cast<const uint16_t*>(b->data), n1 * d,
                           n2 * d, (int32_t)n1, (int32_t)n2, da, db);
    else
        MR_LAUNCH(nce_grad_rows_finish<float>, dim3(grid_1d(n_gt * d), batch), dim3(256), 0, st, r,
                           static_cast<const float*>(a->data), static_cast<const float*>(b->data), n1 * d, n2 * d,
                           (int32_t)n1, (int32_t)n2, da, db);
    if (dev_err()) return MR_ERR_DEVICE;
    const double inv_tau = 1.0 / (double)tau;
    if (n1 > 0)
        MR_LAUNCH(nce_grad_scale, dim3(grid_1d(batch * n1 * d)), dim3(256), 0, st, da, grad_a,
                           (int64_t)batch * n1 * d, inv_tau);
    MR_LAUNCH(nce_grad_scale, dim3(grid_1d(batch * n2 * d)), dim3(256), 0, st, db, grad_b,
                       (int64_t)batch * n2 * d, inv_tau);
    return dev_err();
}

// Device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept; every GPU holds its own copy at its own address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int static_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MR_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MR_ERR_DEVICE;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MR_OK;
}

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
        case MR_ERR_SCRATCH: return "the problem needs more scratch than the static buffer holds";
        default: return "unknown status";
    }
}

int64_t mr_seed_count(int32_t h, int32_t w, int32_t stride, int32_t offset) {
    return seed_count(h, w, stride, offset);
}

size_t mr_workspace_bytes(int op, const mr_map* a, const mr_map* b, int64_t n_q, int32_t stride,
                          int32_t offset) {
    const bool point = op == MR_OP_POINT_NN || op == MR_OP_POINT_MUTUAL_NN || op == MR_OP_POINT_FAST_RECIPROCAL;
    if (validate_for(a, b, point ? M_POINT : M_INNER) != MR_OK) return 0;
    switch (op) {
        case MR_OP_NN_ARGMAX:
        case MR_OP_POINT_NN:
            if (n_q < 0) return 0;
            return nn_layout(a, b, n_q).total;
        case MR_OP_MUTUAL_NN:
        case MR_OP_POINT_MUTUAL_NN:
            return mutual_layout(a, b).total;
        case MR_OP_FAST_RECIPROCAL_GRAPH:
            if (n_q < 1 || n_q > 65535 || seed_count(a->h, a->w, stride, offset) < 0) return 0;
            return graph_ws_bytes(a, (int32_t)n_q, stride, offset);
        case MR_OP_FAST_RECIPROCAL:
        case MR_OP_POINT_FAST_RECIPROCAL: {
            const int64_t ns = seed_count(a->h, a->w, stride, offset);
            if (ns < 0) return 0;
            return fast_layout(a, b, ns).total;
        }
        case MR_OP_INFONCE: {
            NceLayout L;
            if (validate_nce(a, b, n_q) != MR_OK || nce_layout(a, b, n_q, L) != MR_OK) return 0;
            return L.total;
        }
        case MR_OP_INFONCE_BACKWARD: {
            NceGradLayout L;
            if (validate_nce_grad(a, b, n_q) != MR_OK || nce_grad_layout(a, b, n_q, L) != MR_OK) return 0;
            return L.total;
        }
        default: return 0;
    }
}

int mr_infonce_forward(const mr_map* a, const mr_map* b, const int32_t* gt, int64_t n_gt, float tau,
                       float* out_terms, double* out_loss, void* ws, size_t ws_bytes, void* stream) {
    const CallLog lg("mr_infonce_forward", a, b, "n_gt %lld tau %g ws %zu", (long long)n_gt, (double)tau, ws_bytes);
    return lg.done(infonce_impl(a, b, gt, n_gt, tau, out_terms, out_loss, ws, ws_bytes, stream));
}

int mr_infonce_backward(const mr_map* a, const mr_map* b, const int32_t* gt, int64_t n_gt, float tau,
                        float* out_terms, double* out_loss, float* grad_a, float* grad_b, void* ws, size_t ws_bytes,
                        void* stream) {
    const CallLog lg("mr_infonce_backward", a, b, "n_gt %lld tau %g ws %zu", (long long)n_gt, (double)tau, ws_bytes);
    return lg.done(
        infonce_backward_impl(a, b, gt, n_gt, tau, out_terms, out_loss, grad_a, grad_b, ws, ws_bytes, stream));
}

int mr_nn_argmax(const mr_map* q, const mr_map* db, const int32_t* q_idx, int64_t n_q, int32_t* out_idx,
                 float* out_score, void* ws, size_t ws_bytes, void* stream) {
    const CallLog lg("mr_nn_argmax", q, db, "n_q %lld%s ws %zu", (long long)n_q, q_idx ? " (listed)" : "", ws_bytes);
    return lg.done(nn_impl(q, db, q_idx, n_q, out_idx, out_score, ws, ws_bytes, stream, M_INNER));
}

int mr_mutual_nn(const mr_map* a, const mr_map* b, int32_t* nn_ab, int32_t* nn_ba, int32_t* pairs, int64_t cap,
                 int64_t* n_pairs, void* ws, size_t ws_bytes, void* stream) {
    const CallLog lg("mr_mutual_nn", a, b, "cap %lld ws %zu", (long long)cap, ws_bytes);
    return lg.done(mutual_impl(a, b, nn_ab, nn_ba, pairs, cap, n_pairs, ws, ws_bytes, stream, M_INNER));
}

int mr_fast_reciprocal(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset, int32_t max_iters,
                       int32_t* pairs, int64_t cap, int64_t* n_pairs, int32_t* iter_active, void* ws,
                       size_t ws_bytes, void* stream) {
    const CallLog lg("mr_fast_reciprocal", a, b, "stride %d offset %d iters %d cap %lld ws %zu", stride, offset,
                     max_iters, (long long)cap, ws_bytes);
    return lg.done(
        fast_impl(a, b, stride, offset, max_iters, pairs, cap, n_pairs, iter_active, ws, ws_bytes, stream, M_INNER));
}

int mr_fast_reciprocal_static(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset,
                              int32_t max_iters, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                              int32_t* iter_active, void* stream) {
    const CallLog lg("mr_fast_reciprocal_static", a, b, "stride %d offset %d iters %d cap %lld", stride, offset,
                     max_iters, (long long)cap);
    return lg.done([&]() -> int {
        // the same validation order as mr_fast_reciprocal, then the size check against
        // the static buffer before anything is launched
        int rc = validate_for(a, b, M_INNER);
        if (rc) return rc;
        if (stride < 1 || offset < 0 || max_iters < 0) return MR_ERR_PARAM;
        if (!pairs || !n_pairs) return MR_ERR_NULL;
        const int64_t ns = seed_count(a->h, a->w, stride, offset);
        if (cap < ns) return MR_ERR_CAPACITY;
        if (fast_layout(a, b, ns).total > kStaticScratchBytes) return MR_ERR_SCRATCH;
        void* ws = nullptr;
        if ((rc = static_scratch(&ws))) return rc;
        return fast_impl(a, b, stride, offset, max_iters, pairs, cap, n_pairs, iter_active, ws, kStaticScratchBytes,
                         stream, M_INNER);
    }());
}

int mr_point_nn(const mr_map* q, const mr_map* db, const int32_t* q_idx, int64_t n_q, int32_t* out_idx,
                float* out_dist2, void* ws, size_t ws_bytes, void* stream) {
    const CallLog lg("mr_point_nn", q, db, "n_q %lld%s ws %zu", (long long)n_q, q_idx ? " (listed)" : "", ws_bytes);
    return lg.done(nn_impl(q, db, q_idx, n_q, out_idx, out_dist2, ws, ws_bytes, stream, M_POINT));
}

int mr_point_mutual_nn(const mr_map* a, const mr_map* b, int32_t* nn_ab, int32_t* nn_ba, int32_t* pairs,
                       int64_t cap, int64_t* n_pairs, void* ws, size_t ws_bytes, void* stream) {
    const CallLog lg("mr_point_mutual_nn", a, b, "cap %lld ws %zu", (long long)cap, ws_bytes);
    return lg.done(mutual_impl(a, b, nn_ab, nn_ba, pairs, cap, n_pairs, ws, ws_bytes, stream, M_POINT));
}

int mr_point_fast_reciprocal(const mr_map* a, const mr_map* b, int32_t stride, int32_t offset, int32_t max_iters,
                             int32_t* pairs, int64_t cap, int64_t* n_pairs, int32_t* iter_active, void* ws,
                             size_t ws_bytes, void* stream) {
    const CallLog lg("mr_point_fast_reciprocal", a, b, "stride %d offset %d iters %d cap %lld ws %zu", stride, offset,
                     max_iters, (long long)cap, ws_bytes);
    return lg.done(
        fast_impl(a, b, stride, offset, max_iters, pairs, cap, n_pairs, iter_active, ws, ws_bytes, stream, M_POINT));
}

int mr_fast_reciprocal_graph(const mr_map* images, const int32_t* edges, int32_t n_edges, int32_t stride,
                             int32_t offset, int32_t max_iters, int32_t* pairs, int64_t cap, int64_t* n_pairs,
                             int32_t* iter_active, void* ws, size_t ws_bytes, void* stream) {
    const CallLog lg("mr_fast_reciprocal_graph", images, images,
                     "edges %d stride %d offset %d iters %d cap %lld ws %zu", n_edges, stride, offset, max_iters,
                     (long long)cap, ws_bytes);
    return lg.done([&]() -> int {
        int rc = validate_map(images);
        if (rc) return rc;
        if (!edges) return MR_ERR_NULL;
        if (n_edges < 1 || n_edges > 65535) return MR_ERR_PARAM;
        for (int64_t e = 0; e < 2 * (int64_t)n_edges; ++e)
            if (edges[e] < 0 || edges[e] >= images->batch) return MR_ERR_PARAM;
        if (stride < 1 || offset < 0 || max_iters < 0) return MR_ERR_PARAM;
        const mr_map g = graph_map(images, n_edges);
        const size_t at_edges = graph_edges_offset(&g, stride, offset);
        if ((rc = check_ws(ws, ws_bytes, graph_ws_bytes(images, n_edges, stride, offset)))) return rc;
        if (!pairs || !n_pairs) return MR_ERR_NULL;
        if (cap < seed_count(g.h, g.w, stride, offset)) return MR_ERR_CAPACITY;
        hipStream_t st = static_cast<hipStream_t>(stream);
        int32_t* dev_edges = at<int32_t>(ws, at_edges);
        if (hipMemcpyAsync(dev_edges, edges, (size_t)n_edges * 2 * sizeof(int32_t), hipMemcpyHostToDevice, st) !=
            hipSuccess)
            return MR_ERR_DEVICE;
        return fast_impl(&g, &g, stride, offset, max_iters, pairs, cap, n_pairs, iter_active, ws, ws_bytes, stream,
                         M_INNER, dev_edges);
    }());
}

int mr_profile_begin(int32_t max_launches) {
    if (g_prof.on || max_launches < 1) return MR_ERR_PARAM;
    g_prof.ev = static_cast<hipEvent_t*>(calloc((size_t)2 * max_launches, sizeof(hipEvent_t)));
    g_prof.counted = static_cast<bool*>(calloc((size_t)max_launches, sizeof(bool)));
    int made = 0;
    if (g_prof.ev && g_prof.counted)
        while (made < 2 * max_launches && hipEventCreate(&g_prof.ev[made]) == hipSuccess) ++made;
    void* q = nullptr;
    const bool ok = made == 2 * max_launches &&
                    hipMalloc(&q, (size_t)max_launches * sizeof(int64_t)) == hipSuccess;
    if (!ok) {
        for (int k = 0; k < made; ++k) (void)hipEventDestroy(g_prof.ev[k]);
        free(g_prof.ev);
        free(g_prof.counted);
        g_prof = Profiler();
        return MR_ERR_DEVICE;
    }
    g_prof.queries = static_cast<int64_t*>(q);
    g_prof.cap = max_launches;
    g_prof.used = 0;
    g_prof.on = true;
    return MR_OK;
}

int mr_profile_end_queries(double* total_ms, int64_t* launches, float* each_ms, int64_t* each_queries,
                           int32_t cap) {
    if (!g_prof.on || cap < 0 || (cap > 0 && !each_ms && !each_queries)) return MR_ERR_PARAM;
    double tot = 0.0;
    int rc = MR_OK;
    for (int i = 0; i < g_prof.used; ++i) {
        float ms = 0.f;
        if (hipEventSynchronize(g_prof.ev[2 * i + 1]) != hipSuccess ||
            hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]) != hipSuccess)
            rc = MR_ERR_DEVICE;
        tot += ms;
        if (i < cap && each_ms) each_ms[i] = ms;
    }
    const int nq = g_prof.used < cap ? g_prof.used : cap;
    if (each_queries && nq > 0) {
        // the counts were written on the calls' streams, before the end events waited for above
        if (hipMemcpy(each_queries, g_prof.queries, (size_t)nq * sizeof(int64_t), hipMemcpyDeviceToHost) !=
            hipSuccess)
            rc = MR_ERR_DEVICE;
        for (int i = 0; i < nq; ++i)
            if (!g_prof.counted[i]) each_queries[i] = -1;
    }
    for (int i = 0; i < 2 * g_prof.cap; ++i) (void)hipEventDestroy(g_prof.ev[i]);
    free(g_prof.ev);
    free(g_prof.counted);
    (void)hipFree(g_prof.queries);
    if (total_ms) *total_ms = tot;
    if (launches) *launches = g_prof.used;
    g_prof = Profiler();
    return rc;
}

int mr_profile_end_each(double* total_ms, int64_t* launches, float* each_ms, int32_t cap) {
    if (cap > 0 && !each_ms) return MR_ERR_PARAM;
    return mr_profile_end_queries(total_ms, launches, each_ms, nullptr, cap);
}

int mr_profile_end(double* total_ms, int64_t* launches) {
    return mr_profile_end_queries(total_ms, launches, nullptr, nullptr, 0);
}

}  // extern "C"

/* Host-side sanitizer driver for the C ABI of libmr.
 *
 * Linked against a host-only build of the library (no device code, no HIP runtime)
 * made with AddressSanitizer and UndefinedBehaviorSanitizer.  Every HIP function the
 * library imports is defined here as a test double, so nothing needs a GPU:
 *
 *   failing mode     : each HIP call is counted and fails (hipErrorNoDevice);
 *   succeeding mode  : each HIP call is counted and succeeds; a kernel launch records
 *                      its grid, block and LDS size and is checked against gfx950's
 *                      launch limits; nothing is executed.
 *
 * What is checked, beyond the sanitizers' own reports (any report aborts the run):
 *   - every argument error returns its documented status and makes no HIP call
 *     (the header promises validation before anything is launched);
 *   - once a call has made a HIP call, it returns MR_ERR_DEVICE in failing mode and
 *     MR_OK in succeeding mode (no failure is swallowed or invented);
 *   - every launch the host code builds fits the launch limits;
 *   - host buffers the library reads (map descriptors, the graph's edge list) are
 *     read within their bounds: each lives in a heap block of exactly its size;
 *   - a seeded fuzz of descriptors and parameters over every entry point keeps to
 *     the documented status range and the rules above.
 *
 * Usage: abi_driver [fuzz_cases]   -- prints one summary line, exit status 0 on success;
 *        abi_driver overflow       -- a deliberate heap over-read by the library, which
 *                                     AddressSanitizer must report;
 *        abi_driver log            -- valid calls of every entry point, for the launch log.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "mr.h"

/* ------------------------------------------------------------------ HIP test doubles */

typedef struct { uint32_t x, y, z; } dim3_t;

enum { HIP_OK = 0, HIP_NO_DEVICE = 100 };

static int g_fail = 1;         /* 1: every HIP call fails; 0: every HIP call succeeds */
static long g_calls;           /* HIP calls made (registration at load time excluded) */
static long g_launches;        /* kernel launches reaching hipLaunchKernel */
static long g_bad_launches;    /* launches outside the limits */
static dim3_t g_grid, g_block; /* the configuration pushed by the last <<<>>> */
static size_t g_shmem;
static void* g_stream;
static int g_event_id;

static int hip_result(void) { ++g_calls; return g_fail ? HIP_NO_DEVICE : HIP_OK; }

static void* g_module_handle;
void** __hipRegisterFatBinary(const void* data) { (void)data; return &g_module_handle; }
void __hipUnregisterFatBinary(void** modules) { (void)modules; }
void __hipRegisterFunction(void** modules, const void* host_fn, char* dev_fn, const char* dev_name,
                           unsigned int thread_limit, void* tid, void* bid, void* block, void* grid, int* wsize) {
    (void)modules; (void)host_fn; (void)dev_fn; (void)dev_name; (void)thread_limit;
    (void)tid; (void)bid; (void)block; (void)grid; (void)wsize;
}
void __hipRegisterVar(void** modules, void* var, char* host_var, char* dev_var, int ext, size_t size, int constant,
                      int global) {
    (void)modules; (void)var; (void)host_var; (void)dev_var; (void)ext; (void)size; (void)constant; (void)global;
}

int __hipPushCallConfiguration(dim3_t grid, dim3_t block, size_t shmem, void* stream) {
    g_grid = grid; g_block = block; g_shmem = shmem; g_stream = stream;
    return hip_result();
}
int __hipPopCallConfiguration(dim3_t* grid, dim3_t* block, size_t* shmem, void** stream) {
    *grid = g_grid; *block = g_block; *shmem = g_shmem; *stream = g_stream;
    return hip_result();
}
int hipLaunchKernel(const void* fn, dim3_t grid, dim3_t block, void** args, size_t shmem, void* stream) {
    (void)stream;
    ++g_launches;
    const uint64_t threads = (uint64_t)block.x * block.y * block.z;
    const int bad = !fn || !args || grid.x < 1 || grid.y < 1 || grid.z < 1 || block.x < 1 || block.y < 1 ||
                    block.z < 1 || threads > 1024 || grid.x > 2147483647u || grid.y > 65535u || grid.z > 65535u ||
                    (uint64_t)grid.x * block.x > 4294967295ull || shmem > 163840;
    if (bad) {
        ++g_bad_launches;
        fprintf(stderr, "launch outside the limits: grid %u %u %u block %u %u %u lds %zu\n", grid.x, grid.y,
                grid.z, block.x, block.y, block.z, shmem);
    }
    return hip_result();
}
int hipGetLastError(void) { return hip_result(); }
int hipGetDevice(int* dev) {
    int r = hip_result();
    if (!r) *dev = 0;
    return r;
}
/* The device-property struct's layout belongs to the HIP headers; the double always
 * fails this query, so the library takes its default compute-unit count. */
int hipGetDevicePropertiesR0600(void* prop, int dev) { (void)prop; (void)dev; ++g_calls; return HIP_NO_DEVICE; }
int hipOccupancyMaxActiveBlocksPerMultiprocessor(int* n, const void* fn, int block, size_t shmem) {
    (void)fn; (void)block; (void)shmem;
    int r = hip_result();
    if (!r) *n = 2;
    return r;
}
int hipEventCreate(void** ev) {
    int r = hip_result();
    if (!r) *ev = (void*)(uintptr_t)(0x1000 + 16 * ++g_event_id);
    return r;
}
int hipEventDestroy(void* ev) { (void)ev; return hip_result(); }
int hipEventRecord(void* ev, void* stream) { (void)ev; (void)stream; return hip_result(); }
int hipEventSynchronize(void* ev) { (void)ev; return hip_result(); }
int hipEventElapsedTime(float* ms, void* start, void* stop) {
    (void)start; (void)stop;
    int r = hip_result();
    if (!r) *ms = 0.25f;
    return r;
}
static char g_symbol_stand_in[256] __attribute__((aligned(256)));
int hipGetSymbolAddress(void** p, const void* sym) {
    (void)sym;
    int r = hip_result();
    if (!r) *p = g_symbol_stand_in; /* never dereferenced: the launches are doubles too */
    return r;
}
static char g_device_stand_in[4096] __attribute__((aligned(256)));
int hipMalloc(void** p, size_t n) {
    int r = hip_result();
    if (!r) *p = n <= sizeof(g_device_stand_in) ? (void*)g_device_stand_in : (void*)(uintptr_t)(1u << 28);
    return r;
}
int hipFree(void* p) { (void)p; return hip_result(); }
/* the only blocking copy is device -> host of the profiling window's counts: write a
 * recognisable value into every byte of the host side, so that an over-long size shows
 * up as a heap overflow and the caller's use of the values can be checked */
int hipMemcpy(void* dst, const void* src, size_t n, int kind) {
    (void)src; (void)kind;
    int r = hip_result();
    if (!r) memset(dst, 7, n);
    return r;
}
int hipMemcpyAsync(void* dst, const void* src, size_t n, int kind, void* stream) {
    (void)dst; (void)kind; (void)stream;
    /* the only copy the library makes is host -> device of the graph's edges: read the
     * host side in full so that an over-long size shows up as a heap overflow */
    volatile unsigned char sink = 0;
    for (size_t i = 0; i < n; ++i) sink ^= ((const unsigned char*)src)[i];
    (void)sink;
    return hip_result();
}

/* ------------------------------------------------------------------ helpers */

#define FAKE ((void*)(uintptr_t)(1u << 20)) /* aligned device stand-in; never dereferenced */
#define FAKE_WS ((void*)(uintptr_t)(1u << 24))

static long g_cases, g_failures;

/* A descriptor in a heap block of exactly its size. */
static mr_map* mk(int32_t batch, int32_t h, int32_t w, int32_t d, int32_t dtype, const void* data) {
    mr_map* m = (mr_map*)malloc(sizeof(mr_map));
    m->data = data; m->batch = batch; m->h = h; m->w = w; m->d = d; m->dtype = dtype;
    return m;
}
static mr_map* mkd(int32_t batch, int32_t h, int32_t w, int32_t d, int32_t dtype) {
    return mk(batch, h, w, d, dtype, FAKE);
}

/* Check one call's status.  want_hip: 0 = no HIP call allowed, 1 = at least one
 * required, -1 = either. */
static void check(const char* what, int line, int got, int want, long calls_before, int want_hip) {
    ++g_cases;
    const long made = g_calls - calls_before;
    int ok = got == want;
    if (want_hip == 0 && made != 0) ok = 0;
    if (want_hip == 1 && made == 0) ok = 0;
    if (!ok) {
        ++g_failures;
        fprintf(stderr, "FAIL line %d %s: status %d (want %d), HIP calls %ld\n", line, what, got, want, made);
    }
}
#define CHECK(call, want, want_hip)                                  \
    do {                                                             \
        const long c0_ = g_calls;                                    \
        const int r_ = (call);                                       \
        check(#call, __LINE__, r_, (want), c0_, (want_hip));         \
    } while (0)
/* an argument error: the documented status, before any HIP call */
#define REJECT(call, want) CHECK(call, want, 0)
/* a valid call: reaches the device (stub result decides the status) */
#define REACH(call) CHECK(call, g_fail ? MR_ERR_DEVICE : MR_OK, 1)

static void* outp(void) { return FAKE; }

/* ------------------------------------------------------------------ fixed cases */

static void validation_cases(void) {
    void* o = outp();
    /* status strings and seed counts */
    for (int s = 0; s <= 8; ++s) {
        ++g_cases;
        const char* t = mr_status_str(s);
        if (!t || !t[0] || strcmp(t, mr_status_str(99)) == 0) { ++g_failures; fprintf(stderr, "status %d\n", s); }
    }
    ++g_cases;
    if (mr_seed_count(512, 384, 8, 4) != 3072 || mr_seed_count(4, 4, 0, 0) != -1 || mr_seed_count(4, 4, 2, 4) != 0 ||
        mr_seed_count(1 << 14, 1 << 14, 1, 0) != (int64_t)1 << 28) {
        ++g_failures; fprintf(stderr, "seed counts\n");
    }

    /* descriptors: each row is (a, b, status) for both mutual and fast */
    struct { mr_map *a, *b; int want; } rows[] = {
        {NULL, mkd(1, 8, 6, 24, MR_F32), MR_ERR_NULL},
        {mkd(1, 8, 6, 0, MR_F32), mkd(1, 8, 6, 0, MR_F32), MR_ERR_SHAPE},
        {mkd(1, 8, 6, 65, MR_F32), mkd(1, 8, 6, 65, MR_F32), MR_ERR_SHAPE},
        {mkd(1, -1, 6, 24, MR_F32), mkd(1, 8, 6, 24, MR_F32), MR_ERR_SHAPE},
        {mkd(0, 8, 6, 24, MR_F32), mkd(0, 8, 6, 24, MR_F32), MR_ERR_SHAPE},
        {mkd(65536, 8, 6, 24, MR_F32), mkd(65536, 8, 6, 24, MR_F32), MR_ERR_SHAPE},
        {mkd(1, 1 << 15, 1 << 14, 24, MR_F32), mkd(1, 8, 6, 24, MR_F32), MR_ERR_SHAPE},
        {mkd(1, 8, 6, 24, 7), mkd(1, 8, 6, 24, 7), MR_ERR_DTYPE},
        {mkd(1, 8, 6, 12, MR_BF16), mkd(1, 8, 6, 12, MR_BF16), MR_ERR_DTYPE},
        {mkd(1, 8, 6, 24, MR_F32), mkd(1, 8, 6, 24, MR_BF16), MR_ERR_DTYPE},
        {mkd(1, 8, 6, 24, MR_F32), mkd(2, 8, 6, 24, MR_F32), MR_ERR_SHAPE},
        {mkd(1, 8, 6, 24, MR_F32), mkd(1, 8, 6, 16, MR_F32), MR_ERR_SHAPE},
        {mk(1, 8, 6, 24, MR_F32, (char*)FAKE + 4), mkd(1, 8, 6, 24, MR_F32), MR_ERR_SHAPE},
        {mk(1, 8, 6, 24, MR_F32, NULL), mkd(1, 8, 6, 24, MR_F32), MR_ERR_NULL},
    };
    for (size_t i = 0; i < sizeof(rows) / sizeof(rows[0]); ++i) {
        mr_map *a = rows[i].a, *b = rows[i].b;
        REJECT(mr_fast_reciprocal(a, b, 8, 4, 10, o, 1 << 20, o, NULL, FAKE_WS, (size_t)1 << 30, NULL), rows[i].want);
        REJECT(mr_fast_reciprocal_static(a, b, 8, 4, 10, o, 1 << 20, o, NULL, NULL), rows[i].want);
        REJECT(mr_mutual_nn(a, b, o, o, o, 1 << 20, o, FAKE_WS, (size_t)1 << 30, NULL), rows[i].want);
        if (a) {
            ++g_cases;
            if (mr_workspace_bytes(MR_OP_FAST_RECIPROCAL, a, b, 0, 8, 4) != 0) { ++g_failures; fprintf(stderr, "ws row %zu\n", i); }
        }
        free(a); free(b);
    }

    /* the fast scheme's parameters, outputs, capacity and workspace */
    {
        mr_map *a = mkd(1, 64, 48, 24, MR_F32), *b = mkd(1, 64, 48, 24, MR_F32);
        const size_t need = mr_workspace_bytes(MR_OP_FAST_RECIPROCAL, a, b, 0, 8, 4);
        ++g_cases;
        if (need == 0) { ++g_failures; fprintf(stderr, "fast need\n"); }
        REJECT(mr_fast_reciprocal(a, b, 0, 4, 10, o, 48, o, NULL, FAKE_WS, need, NULL), MR_ERR_PARAM);
        REJECT(mr_fast_reciprocal(a, b, 8, -1, 10, o, 48, o, NULL, FAKE_WS, need, NULL), MR_ERR_PARAM);
        REJECT(mr_fast_reciprocal(a, b, 8, 4, -1, o, 48, o, NULL, FAKE_WS, need, NULL), MR_ERR_PARAM);
        REJECT(mr_fast_reciprocal(a, b, 8, 4, 10, NULL, 48, o, NULL, FAKE_WS, need, NULL), MR_ERR_NULL);
        REJECT(mr_fast_reciprocal(a, b, 8, 4, 10, o, 48, NULL, NULL, FAKE_WS, need, NULL), MR_ERR_NULL);
        REJECT(mr_fast_reciprocal(a, b, 8, 4, 10, o, 47, o, NULL, FAKE_WS, need, NULL), MR_ERR_CAPACITY);
        REJECT(mr_fast_reciprocal(a, b, 8, 4, 10, o, 48, o, NULL, NULL, need, NULL), MR_ERR_WORKSPACE);
        REJECT(mr_fast_reciprocal(a, b, 8, 4, 10, o, 48, o, NULL, (char*)FAKE_WS + 64, need, NULL), MR_ERR_WORKSPACE);
        REJECT(mr_fast_reciprocal(a, b, 8, 4, 10, o, 48, o, NULL, FAKE_WS, need - 1, NULL), MR_ERR_WORKSPACE);
        REACH(mr_fast_reciprocal(a, b, 8, 4, 10, o, 48, o, NULL, FAKE_WS, need, NULL));
        REACH(mr_fast_reciprocal(a, b, 8, 4, 10, o, 48, o, o, FAKE_WS, need, NULL));
        REJECT(mr_fast_reciprocal_static(a, b, 0, 4, 10, o, 48, o, NULL, NULL), MR_ERR_PARAM);
        REJECT(mr_fast_reciprocal_static(a, b, 8, 4, 10, o, 47, o, NULL, NULL), MR_ERR_CAPACITY);
        REACH(mr_fast_reciprocal_static(a, b, 8, 4, 10, o, 48, o, NULL, NULL));
        free(a); free(b);
        mr_map *big = mkd(1, 2048, 2048, 24, MR_F32), *ten = mkd(10, 512, 384, 24, MR_F32);
        REJECT(mr_fast_reciprocal_static(big, big, 8, 4, 10, o, 1 << 20, o, NULL, NULL), MR_ERR_SCRATCH);
        REJECT(mr_fast_reciprocal_static(ten, ten, 8, 4, 10, o, 3072, o, NULL, NULL), MR_ERR_SCRATCH);
        free(big); free(ten);
    }

    /* brute-force mutual NN and the NN search */
    {
        mr_map *a = mkd(1, 10, 10, 24, MR_F32), *b = mkd(1, 7, 9, 24, MR_F32);
        const size_t need = mr_workspace_bytes(MR_OP_MUTUAL_NN, a, b, 0, 1, 0);
        REJECT(mr_mutual_nn(a, b, NULL, o, o, 63, o, FAKE_WS, need, NULL), MR_ERR_NULL);
        REJECT(mr_mutual_nn(a, b, o, o, o, 62, o, FAKE_WS, need, NULL), MR_ERR_CAPACITY);
        REJECT(mr_mutual_nn(a, b, o, o, o, 63, o, FAKE_WS, need - 1, NULL), MR_ERR_WORKSPACE);
        REACH(mr_mutual_nn(a, b, o, o, o, 63, o, FAKE_WS, need, NULL));
        const size_t nneed = mr_workspace_bytes(MR_OP_NN_ARGMAX, a, b, 100, 1, 0);
        REJECT(mr_nn_argmax(a, b, NULL, 99, o, NULL, FAKE_WS, nneed, NULL), MR_ERR_PARAM);
        REJECT(mr_nn_argmax(a, b, NULL, -1, o, NULL, FAKE_WS, nneed, NULL), MR_ERR_PARAM);
        REJECT(mr_nn_argmax(a, b, NULL, 100, NULL, NULL, FAKE_WS, nneed, NULL), MR_ERR_NULL);
        REJECT(mr_nn_argmax(a, b, NULL, 100, o, NULL, FAKE_WS, nneed - 8, NULL), MR_ERR_WORKSPACE);
        REACH(mr_nn_argmax(a, b, NULL, 100, o, o, FAKE_WS, nneed, NULL));
        REACH(mr_nn_argmax(a, b, o, 100, o, NULL, FAKE_WS, nneed, NULL));
        CHECK(mr_nn_argmax(a, b, o, 0, NULL, NULL, NULL, 0, NULL), MR_OK, 0); /* nothing to do */
        mr_map* empty = mk(1, 0, 5, 24, MR_F32, NULL);
        REJECT(mr_nn_argmax(empty, b, o, 3, o, NULL, FAKE_WS, (size_t)1 << 20, NULL), MR_ERR_SHAPE);
        free(empty);
        ++g_cases;
        if (mr_workspace_bytes(99, a, b, 0, 1, 0) != 0) { ++g_failures; fprintf(stderr, "op 99\n"); }
        free(a); free(b);
    }

    /* pointmaps */
    {
        mr_map *a = mkd(1, 10, 10, 3, MR_F32), *b = mkd(1, 7, 9, 3, MR_F32);
        mr_map *bf = mkd(1, 10, 10, 8, MR_BF16), *d5 = mkd(1, 10, 10, 5, MR_F32);
        REJECT(mr_point_nn(bf, bf, NULL, 100, o, NULL, FAKE_WS, (size_t)1 << 30, NULL), MR_ERR_DTYPE);
        REJECT(mr_point_mutual_nn(bf, bf, o, o, o, 1 << 20, o, FAKE_WS, (size_t)1 << 30, NULL), MR_ERR_DTYPE);
        REJECT(mr_point_fast_reciprocal(bf, bf, 8, 4, 10, o, 1 << 20, o, NULL, FAKE_WS, (size_t)1 << 30, NULL),
               MR_ERR_DTYPE);
        REJECT(mr_point_nn(d5, d5, NULL, 100, o, NULL, FAKE_WS, (size_t)1 << 30, NULL), MR_ERR_SHAPE);
        REJECT(mr_point_fast_reciprocal(a, b, 8, 4, 10, o, 0, o, NULL, FAKE_WS, (size_t)1 << 30, NULL),
               MR_ERR_CAPACITY);
        REACH(mr_point_nn(a, b, NULL, 100, o, o, FAKE_WS, mr_workspace_bytes(MR_OP_POINT_NN, a, b, 100, 1, 0), NULL));
        REACH(mr_point_mutual_nn(a, b, o, o, o, 63, o, FAKE_WS,
                                 mr_workspace_bytes(MR_OP_POINT_MUTUAL_NN, a, b, 0, 1, 0), NULL));
        REACH(mr_point_fast_reciprocal(a, b, 2, 1, 10, o, 25, o, o, FAKE_WS,
                                       mr_workspace_bytes(MR_OP_POINT_FAST_RECIPROCAL, a, b, 0, 2, 1), NULL));
        free(a); free(b); free(bf); free(d5);
    }

    /* the graph call reads its HOST edge list: each list lives in a block of exactly
     * 2 * n_edges ids, the bad id (if any) last, so a read past it is a heap overflow */
    {
        mr_map* imgs = mkd(4, 8, 6, 24, MR_F32);
        const int32_t good[6] = {0, 1, 1, 3, 2, 0};
        int32_t* e = (int32_t*)malloc(sizeof(good));
        memcpy(e, good, sizeof(good));
        const size_t need = mr_workspace_bytes(MR_OP_FAST_RECIPROCAL_GRAPH, imgs, imgs, 3, 8, 4);
        ++g_cases;
        if (need == 0 || mr_workspace_bytes(MR_OP_FAST_RECIPROCAL_GRAPH, imgs, imgs, 0, 8, 4) != 0) {
            ++g_failures; fprintf(stderr, "graph need\n");
        }
        REJECT(mr_fast_reciprocal_graph(imgs, e, 0, 8, 4, 10, o, 1, o, NULL, FAKE_WS, need, NULL), MR_ERR_PARAM);
        REJECT(mr_fast_reciprocal_graph(imgs, NULL, 3, 8, 4, 10, o, 1, o, NULL, FAKE_WS, need, NULL), MR_ERR_NULL);
        REJECT(mr_fast_reciprocal_graph(imgs, e, 3, 8, 4, 10, o, 1, o, NULL, FAKE_WS, need - 1, NULL),
               MR_ERR_WORKSPACE);
        REJECT(mr_fast_reciprocal_graph(imgs, e, 3, 8, 4, 10, o, 0, o, NULL, FAKE_WS, need, NULL), MR_ERR_CAPACITY);
        REACH(mr_fast_reciprocal_graph(imgs, e, 3, 8, 4, 10, o, 1, o, o, FAKE_WS, need, NULL));
        e[5] = 4; /* image 4 of 4, in the last slot */
        REJECT(mr_fast_reciprocal_graph(imgs, e, 3, 8, 4, 10, o, 1, o, NULL, FAKE_WS, need, NULL), MR_ERR_PARAM);
        e[5] = -1;
        REJECT(mr_fast_reciprocal_graph(imgs, e, 3, 8, 4, 10, o, 1, o, NULL, FAKE_WS, need, NULL), MR_ERR_PARAM);
        free(e);
        /* the largest edge count */
        const int32_t ne = 65535;
        int32_t* big = (int32_t*)malloc((size_t)ne * 2 * sizeof(int32_t));
        for (int32_t k = 0; k < 2 * ne; ++k) big[k] = (k * 7 + k / 2) & 3;
        const size_t bneed = mr_workspace_bytes(MR_OP_FAST_RECIPROCAL_GRAPH, imgs, imgs, ne, 8, 4);
        REACH(mr_fast_reciprocal_graph(imgs, big, ne, 8, 4, 10, o, 1, o, o, FAKE_WS, bneed, NULL));
        REJECT(mr_fast_reciprocal_graph(imgs, big, ne + 1, 8, 4, 10, o, 1, o, NULL, FAKE_WS, bneed, NULL),
               MR_ERR_PARAM);
        big[2 * ne - 1] = 4;
        REJECT(mr_fast_reciprocal_graph(imgs, big, ne, 8, 4, 10, o, 1, o, NULL, FAKE_WS, bneed, NULL), MR_ERR_PARAM);
        free(big);
        free(imgs);
    }

    /* the matching loss and its gradient */
    {
        mr_map *a = mkd(1, 10, 10, 24, MR_F32), *b = mkd(1, 7, 9, 24, MR_F32);
        const size_t need = mr_workspace_bytes(MR_OP_INFONCE, a, b, 50, 0, 0);
        const float bad_tau[4] = {0.0f, -0.1f, INFINITY, NAN};
        for (int k = 0; k < 4; ++k)
            REJECT(mr_infonce_forward(a, b, o, 50, bad_tau[k], o, o, FAKE_WS, need, NULL), MR_ERR_PARAM);
        REJECT(mr_infonce_forward(a, b, o, -1, 0.1f, o, o, FAKE_WS, need, NULL), MR_ERR_PARAM);
        REJECT(mr_infonce_forward(a, b, o, ((int64_t)1 << 28) + 1, 0.1f, o, o, FAKE_WS, need, NULL), MR_ERR_PARAM);
        REJECT(mr_infonce_forward(a, b, NULL, 50, 0.1f, o, o, FAKE_WS, need, NULL), MR_ERR_NULL);
        REJECT(mr_infonce_forward(a, b, o, 50, 0.1f, NULL, o, FAKE_WS, need, NULL), MR_ERR_NULL);
        REJECT(mr_infonce_forward(a, b, o, 50, 0.1f, o, NULL, FAKE_WS, need, NULL), MR_ERR_NULL);
        REJECT(mr_infonce_forward(a, b, o, 50, 0.1f, o, o, FAKE_WS, need - 1, NULL), MR_ERR_WORKSPACE);
        REACH(mr_infonce_forward(a, b, o, 50, 0.1f, o, o, FAKE_WS, need, NULL));
        mr_map *a20 = mkd(1, 10, 10, 20, MR_F32), *b20 = mkd(1, 7, 9, 20, MR_F32);
        REJECT(mr_infonce_forward(a20, b20, o, 50, 0.1f, o, o, FAKE_WS, need, NULL), MR_ERR_SHAPE);
        mr_map* b0 = mk(1, 0, 9, 24, MR_F32, NULL);
        REJECT(mr_infonce_forward(a, b0, o, 50, 0.1f, o, o, FAKE_WS, need, NULL), MR_ERR_SHAPE);
        mr_map *ga = mkd(1, 10, 10, 24, MR_BF16), *gb = mkd(1, 7, 9, 24, MR_BF16);
        const size_t gneed = mr_workspace_bytes(MR_OP_INFONCE_BACKWARD, ga, gb, 50, 0, 0);
        REJECT(mr_infonce_backward(a, gb, o, 50, 0.1f, o, o, o, o, FAKE_WS, gneed, NULL), MR_ERR_DTYPE);
        REJECT(mr_infonce_backward(ga, gb, o, 50, 0.1f, o, o, NULL, o, FAKE_WS, gneed, NULL), MR_ERR_NULL);
        REJECT(mr_infonce_backward(ga, gb, o, 50, 0.1f, o, o, o, NULL, FAKE_WS, gneed, NULL), MR_ERR_NULL);
        REJECT(mr_infonce_backward(ga, gb, o, 50, 0.1f, o, o, o, o, FAKE_WS, gneed - 1, NULL), MR_ERR_WORKSPACE);
        REACH(mr_infonce_backward(ga, gb, o, 50, 0.1f, o, o, o, o, FAKE_WS, gneed, NULL));
        REACH(mr_infonce_backward(a, b, o, 50, 0.1f, o, o, o, o, FAKE_WS,
                                  mr_workspace_bytes(MR_OP_INFONCE_BACKWARD, a, b, 50, 0, 0), NULL));
        free(a); free(b); free(a20); free(b20); free(b0); free(ga); free(gb);
    }

    /* the profiling window: begin fails cleanly when events cannot be made, and an
     * end without a begin is a parameter error */
    {
        double ms = -1;
        int64_t n = -1;
        float each[4];
        REJECT(mr_profile_end(&ms, &n), MR_ERR_PARAM);
        REJECT(mr_profile_end_each(&ms, &n, each, 4), MR_ERR_PARAM);
        REJECT(mr_profile_begin(0), MR_ERR_PARAM);
        if (g_fail) {
            CHECK(mr_profile_begin(8), MR_ERR_DEVICE, 1);
            REJECT(mr_profile_end(&ms, &n), MR_ERR_PARAM); /* no window was opened */
        } else {
            CHECK(mr_profile_begin(3), MR_OK, 1);
            REJECT(mr_profile_begin(3), MR_ERR_PARAM); /* one window per thread */
            REJECT(mr_profile_end_each(&ms, &n, NULL, 2), MR_ERR_PARAM);
            mr_map *a = mkd(1, 32, 32, 24, MR_F32), *b = mkd(1, 32, 32, 24, MR_F32);
            const size_t need = mr_workspace_bytes(MR_OP_NN_ARGMAX, a, b, 1024, 1, 0);
            for (int k = 0; k < 5; ++k) REACH(mr_nn_argmax(a, b, NULL, 1024, FAKE, NULL, FAKE_WS, need, NULL));
            CHECK(mr_profile_end_each(&ms, &n, each, 4), MR_OK, 1);
            ++g_cases;
            /* five calls, one search launch each, three of them timed */
            if (n != 3 || ms != 0.75 || each[0] != 0.25f || each[2] != 0.25f) {
                ++g_failures; fprintf(stderr, "profile window: %ld launches, %g ms\n", (long)n, ms);
            }
            /* per-launch query counts: three counted launches, copied into a block of
             * exactly three entries (the double writes 0x0707... into each) */
            CHECK(mr_profile_begin(3), MR_OK, 1);
            for (int k = 0; k < 2; ++k) REACH(mr_nn_argmax(a, b, NULL, 1024, FAKE, NULL, FAKE_WS, need, NULL));
            int64_t* qs = (int64_t*)malloc(3 * sizeof(int64_t));
            qs[2] = -5;
            CHECK(mr_profile_end_queries(&ms, &n, NULL, qs, 3), MR_OK, 1);
            ++g_cases;
            if (n != 2 || qs[0] != 0x0707070707070707ll || qs[1] != qs[0] || qs[2] != -5) {
                ++g_failures; fprintf(stderr, "profile counts: %ld launches\n", (long)n);
            }
            REJECT(mr_profile_end_queries(&ms, &n, NULL, qs, 3), MR_ERR_PARAM); /* closed */
            free(qs);
            free(a); free(b);
        }
    }
}

/* ------------------------------------------------------------------ fuzz */

static uint64_t g_rng = 0x9e3779b97f4a7c15ull;
static uint64_t next_u64(void) { /* splitmix64 */
    uint64_t z = (g_rng += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}
static int pick(int n) { return (int)(next_u64() % (uint64_t)n); }
#define PICK(arr) ((arr)[pick((int)(sizeof(arr) / sizeof((arr)[0])))])

static void fuzz_one(void) {
    static const int32_t batches[] = {1, 1, 2, 3, 8, 16, 64, 1000, 65535, 0, -1, 65536};
    static const int32_t sides[] = {0, 1, 2, 5, 31, 32, 33, 64, 100, 384, 512, 768, 1024, 8192, 16384, -1, 1 << 15};
    static const int32_t ds[] = {1, 2, 3, 4, 8, 16, 20, 24, 32, 40, 64, 0, 5, 65};
    static const int32_t strides[] = {1, 2, 4, 8, 8, 16, 1000, 0, -1};
    static const int32_t iters[] = {0, 1, 10, 10, 1000, -1};
    const int op = pick(12);
    const int point = op == 3 || op == 4 || op == 5;
    const int32_t batch = PICK(batches);
    const int32_t d = point ? 1 + pick(5) : PICK(ds);
    const int32_t dt = point ? (pick(8) ? MR_F32 : MR_BF16) : (pick(9) ? pick(2) : 7);
    int32_t h1 = PICK(sides), w1 = PICK(sides), h2 = PICK(sides), w2 = PICK(sides);
    /* keep most maps under the pixel limit so that calls get past validation */
    while (pick(4) && (int64_t)h1 * w1 > ((int64_t)1 << 24)) { h1 /= 2; w1 /= 2; }
    while (pick(4) && (int64_t)h2 * w2 > ((int64_t)1 << 24)) { h2 /= 2; w2 /= 2; }
    const void* da = pick(16) ? FAKE : (pick(2) ? NULL : (char*)FAKE + 4);
    const void* db = pick(16) ? FAKE : (pick(2) ? NULL : (char*)FAKE + 8);
    mr_map* a = mk(batch, h1, w1, d, dt, da);
    mr_map* b = mk(pick(10) ? batch : PICK(batches), h2, w2, pick(10) ? d : PICK(ds), pick(12) ? dt : 1 - dt, db);
    const int32_t stride = PICK(strides), offset = pick(10) ? pick(stride > 0 ? stride : 1) : -1;
    const int32_t T = PICK(iters);
    const int64_t na = (int64_t)h1 * w1, nb = (int64_t)h2 * w2;
    int64_t nq = pick(6) ? na : (int64_t)pick(3000) - 1;
    const int64_t ngt = pick(8) ? (int64_t)pick(5000) : -1;
    const float tau = pick(10) ? 0.07f : (pick(2) ? 0.0f : NAN);
    static const int ws_ops[12] = {MR_OP_NN_ARGMAX, MR_OP_MUTUAL_NN, MR_OP_FAST_RECIPROCAL, MR_OP_POINT_NN,
                                   MR_OP_POINT_MUTUAL_NN, MR_OP_POINT_FAST_RECIPROCAL, MR_OP_FAST_RECIPROCAL,
                                   MR_OP_FAST_RECIPROCAL_GRAPH, MR_OP_INFONCE, MR_OP_INFONCE_BACKWARD,
                                   MR_OP_NN_ARGMAX, MR_OP_MUTUAL_NN};
    const int32_t ne = pick(8) ? 1 + pick(100) : (pick(2) ? 0 : 65536);
    const int64_t q_arg = op == 7 ? ne : (op == 8 || op == 9) ? ngt : nq;
    const size_t need = mr_workspace_bytes(ws_ops[op], a, op == 7 ? a : b, q_arg, stride, offset);
    size_t wsb = need;
    switch (pick(8)) {
        case 0: wsb = need ? need - 1 : 0; break;
        case 1: wsb = (size_t)-1; break;
        default: break;
    }
    void* ws = pick(16) ? FAKE_WS : (pick(2) ? NULL : (char*)FAKE_WS + 128);
    const int64_t ns = mr_seed_count(op == 7 ? h1 : h1, w1, stride, offset);
    int64_t cap;
    switch (pick(6)) {
        case 0: cap = -1; break;
        case 1: cap = (op == 1 || op == 4 || op == 11) ? (na < nb ? na : nb) - 1 : ns - 1; break;
        default: cap = (int64_t)1 << 40; break;
    }
    void* o = pick(24) ? FAKE : NULL;
    void* o2 = pick(24) ? FAKE : NULL;
    const int32_t* qidx = pick(3) ? NULL : (const int32_t*)FAKE;
    if (qidx == NULL && pick(6)) nq = na;
    int32_t* edges = NULL;
    if (op == 7 && ne > 0 && ne <= 65536) {
        edges = (int32_t*)malloc((size_t)ne * 2 * sizeof(int32_t));
        for (int32_t k = 0; k < 2 * ne; ++k) edges[k] = batch > 0 ? pick(batch) : 0;
        if (!pick(6)) edges[2 * ne - 1] = pick(2) ? batch : -1;
    }

    const long c0 = g_calls, l0 = g_launches;
    int rc = -1;
    switch (op) {
        case 0: rc = mr_nn_argmax(a, b, qidx, nq, o, pick(2) ? o2 : NULL, ws, wsb, NULL); break;
        case 1: rc = mr_mutual_nn(a, b, o, o2, FAKE, cap, FAKE, ws, wsb, NULL); break;
        case 2: rc = mr_fast_reciprocal(a, b, stride, offset, T, o, cap, o2, pick(2) ? FAKE : NULL, ws, wsb, NULL); break;
        case 3: rc = mr_point_nn(a, b, qidx, nq, o, pick(2) ? o2 : NULL, ws, wsb, NULL); break;
        case 4: rc = mr_point_mutual_nn(a, b, o, o2, FAKE, cap, FAKE, ws, wsb, NULL); break;
        case 5: rc = mr_point_fast_reciprocal(a, b, stride, offset, T, o, cap, o2, NULL, ws, wsb, NULL); break;
        case 6: rc = mr_fast_reciprocal_static(a, b, stride, offset, T, o, cap, o2, pick(2) ? FAKE : NULL, NULL); break;
        case 7: rc = mr_fast_reciprocal_graph(a, edges, ne, stride, offset, T, o, cap, o2, NULL, ws, wsb, NULL); break;
        case 8: rc = mr_infonce_forward(a, b, (const int32_t*)o, ngt, tau, o2, FAKE, ws, wsb, NULL); break;
        case 9: rc = mr_infonce_backward(a, b, (const int32_t*)FAKE, ngt, tau, FAKE, FAKE, o, o2, ws, wsb, NULL); break;
        case 10: rc = mr_nn_argmax(b, a, NULL, nb, o, NULL, ws, mr_workspace_bytes(MR_OP_NN_ARGMAX, b, a, nb, 1, 0), NULL); break;
        default: rc = mr_mutual_nn(b, a, o, o2, FAKE, cap, FAKE, ws, wsb, NULL); break;
    }
    const long made = g_calls - c0, launched = g_launches - l0;
    ++g_cases;
    int ok = rc >= MR_OK && rc <= MR_ERR_SCRATCH;
    if (made == 0 && rc == MR_ERR_DEVICE) ok = 0;          /* a device error needs a device call */
    if (made > 0 && rc != (g_fail ? MR_ERR_DEVICE : MR_OK)) ok = 0; /* errors surface, none invented */
    if (launched > 0 && g_fail) ok = 0;                    /* a failed push launches nothing */
    if (!ok) {
        ++g_failures;
        fprintf(stderr, "FUZZ op %d: status %d, HIP calls %ld, launches %ld; a=(%d,%d,%d,%d,%d) b=(%d,%d,%d,%d,%d) "
                        "stride %d offset %d T %d nq %lld ngt %lld cap %lld ws_bytes %zu need %zu\n",
                op, rc, made, launched, a->batch, a->h, a->w, a->d, a->dtype, b->batch, b->h, b->w, b->d, b->dtype,
                stride, offset, T, (long long)nq, (long long)ngt, (long long)cap, wsb, need);
    }
    free(edges);
    free(a);
    free(b);
}

/* A caller error on purpose: the edge list holds 3 edges and the call declares 4, so
 * the library's validation reads past the heap block.  AddressSanitizer must report it
 * (run by the test to show that the library's host code is instrumented). */
static int overflow_control(void) {
    mr_map* imgs = mkd(4, 8, 6, 24, MR_F32);
    int32_t* e = (int32_t*)malloc(6 * sizeof(int32_t));
    for (int k = 0; k < 6; ++k) e[k] = k & 3;
    const int rc = mr_fast_reciprocal_graph(imgs, e, 4, 8, 4, 10, FAKE, 1, FAKE, NULL, FAKE_WS, (size_t)1 << 30,
                                            NULL);
    printf("overflow control returned %d without a report\n", rc);
    free(e);
    free(imgs);
    return 0;
}

/* Valid calls of every entry point with succeeding HIP doubles, for the launch log
 * (MR_LOG): prints how many calls and launches were made, so that the log's lines can
 * be counted against them. */
static int log_calls(void) {
    g_fail = 0;
    void* o = FAKE;
    long calls = 0;
    const long l0 = g_launches;
    mr_map *a = mkd(1, 40, 30, 24, MR_F32), *b = mkd(1, 36, 28, 24, MR_F32);
    mr_map *ha = mkd(1, 40, 30, 24, MR_BF16), *hb = mkd(1, 36, 28, 24, MR_BF16);
    mr_map *pa = mkd(1, 40, 30, 3, MR_F32), *pb = mkd(1, 36, 28, 3, MR_F32), *imgs = mkd(3, 40, 30, 24, MR_F32);
    int rc = 0;
#define LOGGED(call) do { rc |= (call); ++calls; } while (0)
    LOGGED(mr_nn_argmax(a, b, NULL, 1200, o, o, FAKE_WS, mr_workspace_bytes(MR_OP_NN_ARGMAX, a, b, 1200, 1, 0), NULL));
    LOGGED(mr_mutual_nn(a, b, o, o, o, 1008, o, FAKE_WS, mr_workspace_bytes(MR_OP_MUTUAL_NN, a, b, 0, 1, 0), NULL));
    LOGGED(mr_mutual_nn(ha, hb, o, o, o, 1008, o, FAKE_WS, mr_workspace_bytes(MR_OP_MUTUAL_NN, ha, hb, 0, 1, 0), NULL));
    LOGGED(mr_fast_reciprocal(a, b, 8, 4, 10, o, 20, o, o, FAKE_WS,
                              mr_workspace_bytes(MR_OP_FAST_RECIPROCAL, a, b, 0, 8, 4), NULL));
    LOGGED(mr_fast_reciprocal_static(a, b, 8, 4, 10, o, 20, o, o, NULL));
    LOGGED(mr_point_nn(pa, pb, NULL, 1200, o, o, FAKE_WS, mr_workspace_bytes(MR_OP_POINT_NN, pa, pb, 1200, 1, 0), NULL));
    LOGGED(mr_point_mutual_nn(pa, pb, o, o, o, 1008, o, FAKE_WS,
                              mr_workspace_bytes(MR_OP_POINT_MUTUAL_NN, pa, pb, 0, 1, 0), NULL));
    LOGGED(mr_point_fast_reciprocal(pa, pb, 8, 4, 10, o, 20, o, NULL, FAKE_WS,
                                    mr_workspace_bytes(MR_OP_POINT_FAST_RECIPROCAL, pa, pb, 0, 8, 4), NULL));
    int32_t* e = (int32_t*)malloc(4 * sizeof(int32_t));
    e[0] = 0; e[1] = 1; e[2] = 2; e[3] = 0;
    LOGGED(mr_fast_reciprocal_graph(imgs, e, 2, 8, 4, 10, o, 20, o, NULL, FAKE_WS,
                                    mr_workspace_bytes(MR_OP_FAST_RECIPROCAL_GRAPH, imgs, imgs, 2, 8, 4), NULL));
    LOGGED(mr_infonce_forward(ha, hb, o, 100, 0.1f, o, o, FAKE_WS, mr_workspace_bytes(MR_OP_INFONCE, ha, hb, 100, 0, 0),
                              NULL));
    LOGGED(mr_infonce_backward(ha, hb, o, 100, 0.1f, o, o, o, o, FAKE_WS,
                               mr_workspace_bytes(MR_OP_INFONCE_BACKWARD, ha, hb, 100, 0, 0), NULL));
    LOGGED(mr_nn_argmax(a, b, NULL, 7, o, NULL, FAKE_WS, 0, NULL)); /* an argument error: no launch */
#undef LOGGED
    printf("calls %ld launches %ld status_or %d\n", calls, g_launches - l0, rc);
    free(e); free(a); free(b); free(ha); free(hb); free(pa); free(pb); free(imgs);
    return 0;
}

int main(int argc, char** argv) {
    if (argc > 1 && strcmp(argv[1], "overflow") == 0) return overflow_control();
    if (argc > 1 && strcmp(argv[1], "log") == 0) return log_calls();
    const long fuzz = argc > 1 ? atol(argv[1]) : 4000;
    long reached[2] = {0, 0};
    for (int mode = 1; mode >= 0; --mode) {
        g_fail = mode;
        const long c0 = g_calls;
        validation_cases();
        for (long k = 0; k < fuzz; ++k) fuzz_one();
        reached[mode] = g_calls - c0;
    }
    if (g_bad_launches) ++g_failures;
    printf("cases %ld failures %ld launches %ld bad_launches %ld hip_calls_failing %ld hip_calls_succeeding %ld\n",
           g_cases, g_failures, g_launches, g_bad_launches, reached[1], reached[0]);
    return g_failures ? 1 : 0;
}

// os_abi.hip -- the C ABI declared in include/online_softmax.h: argument
// checks (all before any HIP call), kernel selection, and launches on the
// caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>


#include "../../include/online_softmax.h"
#include "os_kernels.hpp"
#include "os_attention.hpp"

using namespace onorm;

namespace {

constexpr int kVersion = 200;  // 0.2.0: logsumexp, split-row forward, bf16 top-K, row-pattern copy

thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof g_error, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_error[0] = '\0';
    return OS_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int elt_size(int dtype) { return dtype == OS_BF16 ? 2 : 4; }

// Workspaces hold a fixed number of bytes per (row, slice); refuse row counts
// whose workspace size would not fit in int64 (with room for alignment).
constexpr int64_t kMaxWorkspaceBytes = int64_t(1) << 60;
bool workspace_fits(int64_t rows, int64_t bytes_per_row) { return rows <= kMaxWorkspaceBytes / bytes_per_row; }

// Common checks of a [rows, cols] problem.  Returns OS_OK, an error, or 1 for
// "empty: nothing to do".
int check_problem(const char* fn, const void* in, const void* out, bool need_out, int64_t rows,
                  int64_t cols, int dtype) {
    if (dtype != OS_F32 && dtype != OS_BF16) return fail(OS_EINVAL, "%s: unknown dtype %d", fn, dtype);
    if (rows < 0 || cols < 0)
        return fail(OS_EINVAL, "%s: rows (%lld) and cols (%lld) must be >= 0", fn, (long long)rows,
                    (long long)cols);
    if (cols > OS_MAX_COLS) return fail(OS_EINVAL, "%s: cols %lld exceeds OS_MAX_COLS", fn, (long long)cols);
    if (rows == 0 || cols == 0) return 1;
    if (rows > INT64_MAX / cols / 4)
        return fail(OS_EINVAL, "%s: rows * cols overflows the addressable range", fn);
    if (in == nullptr) return fail(OS_EINVAL, "%s: input pointer is NULL", fn);
    if (need_out && out == nullptr) return fail(OS_EINVAL, "%s: output pointer is NULL", fn);
    const uintptr_t es = static_cast<uintptr_t>(elt_size(dtype));
    if (!aligned(in, es) || (out != nullptr && !aligned(out, es)))
        return fail(OS_EINVAL, "%s: pointers must be aligned to the element size (%d bytes)", fn,
                    (int)es);
    return OS_OK;
}

// 16-byte vector path: every row start aligned (base aligned, row bytes a multiple of 16).
bool vector_ok(const void* in, const void* out, int64_t cols, int dtype) {
    return aligned(in, 16) && (out == nullptr || aligned(out, 16)) && ((cols * elt_size(dtype)) % 16) == 0;
}

int launched(const char* fn) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(OS_ELAUNCH, "%s: launch failed: %s", fn, hipGetErrorString(e));
    return ok();
}

// ---------------------------------------------------------------------------
// Register-resident shapes built into the library.
// ---------------------------------------------------------------------------
typedef void (*RowKernel)(const void*, void*, RowStats, int64_t, int, uint32_t);
typedef void (*SafeKernel)(const void*, void*, int64_t, int, uint32_t, int);

struct ResidentShape {
    int lpr, vpl;
    RowKernel fn[2][2];     // [bf16][aligned]
    SafeKernel safe[2][2];  // the three-pass baseline with the same geometry
    RowKernel staged[2];    // [bf16]: rows not 16-byte aligned, read and written through LDS (lpr <= 64)
    RowKernel dense;        // fp32 aligned rows at 8 waves per SIMD, for small batches (see dense_rows)
};

// fp32 rows on 512 or 1024 lanes of 8 vectors take 74-77 VGPRs, which leaves
// room for one 1024-lane (three 512-lane) workgroups per CU; the same kernel
// held to 64 VGPRs fits two (four), without spilling.  On large batches that
// measured 0.4-2% slower (4096 x 32000: 176.6 us against 172.7), but a batch
// of at most two such rounds of workgroups starts in fewer rounds and ends
// sooner: 300 x 32000 takes 15.6 us instead of 16.6, 1000 x 32000 44.5 us
// instead of 46.0.
template <int L, int V>
constexpr RowKernel dense_kernel() {
    if constexpr (L >= 512 && V == 8) return k_resident<false, L, V, true, 0, 8>;
    else return nullptr;
}

// Largest number of workgroups that takes the dense kernel: two rounds of
// them over MI355X's 256 CUs at 32 waves per CU.
constexpr int64_t dense_rows(int block) { return 2 * 256 * (32 * 64 / block); }

// Multi-row shapes may read rows that are not 16-byte aligned through LDS
// (where the plan says so: see the plan tables and plan_for).
template <bool BF16, int L, int V>
constexpr RowKernel staged_kernel() {
    if constexpr (L <= 64) return k_resident<BF16, L, V, false, 2>;
    else return nullptr;
}

// Multi-row shapes (L <= 64) on rows that are not 16-byte aligned assemble
// each workgroup's run of output rows in LDS and store it as whole 16-byte
// blocks (measured 2-60% faster than per-slot stores with the rows' partial
// end slots written element by element; bitwise the same results).
#define ONORM_RESIDENT(L, V)                                                         \
    {                                                                                \
        L, V,                                                                        \
            {                                                                        \
                {k_resident<false, L, V, false, (L <= 64 ? 1 : 0)>, k_resident<false, L, V, true, 0>}, \
                {k_resident<true, L, V, false, (L <= 64 ? 1 : 0)>, k_resident<true, L, V, true, 0>},   \
            },                                                                       \
        {                                                                            \
            {k_safe3_rows<false, L, V, false>, k_safe3_rows<false, L, V, true>},     \
                {k_safe3_rows<true, L, V, false>, k_safe3_rows<true, L, V, true>},   \
        },                                                                           \
        {staged_kernel<false, L, V>(), staged_kernel<true, L, V>()},                 \
        dense_kernel<L, V>()                                                         \
    }
// fp32 only: 16 vectors of bf16 are 128 fp32 values per lane, more than a
// 1024-thread workgroup's 128-VGPR budget, so bf16 rows this long stream.
// No three-pass form: the baseline streams rows this long.
#define ONORM_RESIDENT_F32(L, V)                                                     \
    {                                                                                \
        L, V,                                                                        \
            {                                                                        \
                {k_resident<false, L, V, false, 0>, k_resident<false, L, V, true, 0>},     \
                {nullptr, nullptr},                                                  \
            },                                                                       \
        {                                                                            \
            {nullptr, nullptr},                                                      \
                {nullptr, nullptr},                                                  \
        },                                                                           \
        {nullptr, nullptr},                                                          \
        nullptr                                                                      \
    }

constexpr ResidentShape kResident[] = {
    ONORM_RESIDENT(4, 1),     ONORM_RESIDENT(4, 2),     ONORM_RESIDENT(4, 4),
    ONORM_RESIDENT(8, 1),     ONORM_RESIDENT(8, 2),     ONORM_RESIDENT(8, 4),
    ONORM_RESIDENT(16, 1),    ONORM_RESIDENT(16, 2),    ONORM_RESIDENT(16, 4),
    ONORM_RESIDENT(32, 1),    ONORM_RESIDENT(32, 2),    ONORM_RESIDENT(32, 4),
    ONORM_RESIDENT(64, 1),    ONORM_RESIDENT(64, 2),    ONORM_RESIDENT(64, 4),    ONORM_RESIDENT(64, 8),
    ONORM_RESIDENT(128, 1),   ONORM_RESIDENT(128, 2),   ONORM_RESIDENT(128, 4),   ONORM_RESIDENT(128, 8),
    ONORM_RESIDENT(256, 1),   ONORM_RESIDENT(256, 2),   ONORM_RESIDENT(256, 4),   ONORM_RESIDENT(256, 8),
    ONORM_RESIDENT(512, 1),   ONORM_RESIDENT(512, 2),   ONORM_RESIDENT(512, 4),   ONORM_RESIDENT(512, 8),
    ONORM_RESIDENT(1024, 1),  ONORM_RESIDENT(1024, 2),  ONORM_RESIDENT(1024, 4),  ONORM_RESIDENT(1024, 8),
    // rows just past a power of two in slots (a lane at 5 or 6 vectors)
    ONORM_RESIDENT(256, 5),   ONORM_RESIDENT(512, 5),   ONORM_RESIDENT(512, 6),   ONORM_RESIDENT(1024, 5),
    ONORM_RESIDENT(1024, 6),  ONORM_RESIDENT(1024, 7),
    ONORM_RESIDENT_F32(1024, 16),
};
constexpr int kNumResident = sizeof(kResident) / sizeof(kResident[0]);

// Automatic choice, by the number of 16-byte slots a row spans, from sweeps
// of every built shape on MI355X at ~0.5 GiB per launch: 90 lengths per
// table (rows at both ends and in the middle of every power-of-two bucket of
// slots, and lengths that leave 0-7 slots spare on 256-1024 lanes), 96 rows
// one element short of a whole number of blocks and 96 random lengths.
// Entry {n, l, v, s} serves rows of up to n slots with l lanes of v vectors,
// read through LDS when s is set.  Over those 552 lengths the choice (with
// plan_for's rule) averages 0.2-0.4% above the best shape for each length (a
// geometric mean; the worst single length is 6% above it).
//  - A row just past a power of two often runs fastest on half the lanes with
//    twice the vectors (smaller workgroups, or more rows per wavefront), and
//    past 1024, 2048 and 4096 slots on 5, 6 or 7 vectors per lane (rows of
//    1-25% past the power of two measured 2-20% faster than on 8 vectors).
//  - One-row shapes (over 64 lanes) keep 8 or more slots spare on rows that
//    are not 16-byte aligned, and fp32 rows past 4096 slots, so that the
//    workgroup may start at the 128-byte line holding the row: at 0-7 spare
//    slots it starts at the row's 16-byte block, measured 3-8% slower (e.g.
//    16381 fp32 columns on 1024 x 4 in 184.7 us against 175 us on 1024 x 5).
//  - Short fp32 rows that are not 16-byte aligned run fastest read through
//    LDS (5-32 slots: 166-173 us against 174-262 us for the best direct
//    loads, 9 slots 1.5x); bf16 rows measured faster with direct loads at
//    every length but one, and keep them.
struct PlanEntry {
    int max_slots, lpr, vpl;
    bool staged;
};
constexpr PlanEntry kPlanF32[] = {
    {4, 4, 1},        {8, 8, 1},        {16, 16, 1},      {24, 16, 2},      {32, 32, 1},      {48, 32, 2},
    {64, 64, 1},      {128, 64, 2},     {256, 128, 2},    {512, 256, 2},    {560, 256, 4},    {640, 256, 5},
    {1024, 512, 2},   {1152, 512, 4},   {1280, 512, 5},   {1408, 512, 6},   {2048, 512, 8},   {3072, 1024, 4},
    {5112, 1024, 6},  {7160, 1024, 7},  {8192, 1024, 8}};
constexpr PlanEntry kPlanF32Unaligned[] = {
    {4, 4, 1},        {8, 4, 2, true},  {10, 4, 4, true}, {16, 8, 2, true}, {32, 8, 4, true}, {36, 16, 4, true},
    {40, 32, 2},      {56, 32, 4},      {64, 64, 1},      {68, 32, 4, true}, {128, 64, 2},    {216, 64, 4, true},
    {288, 64, 8},     {352, 64, 8, true}, {504, 256, 2},  {960, 256, 4},    {1152, 256, 5},   {1920, 256, 8},
    {2304, 512, 6},   {4088, 1024, 4},  {5112, 1024, 5},  {6136, 1024, 6},  {7160, 1024, 7},  {8192, 1024, 8}};
constexpr PlanEntry kPlanBF16[] = {
    {4, 4, 1},        {8, 8, 1},        {16, 16, 1},      {24, 16, 2},      {32, 32, 1},      {64, 32, 2},
    {128, 64, 2},     {224, 64, 4},     {256, 128, 2},    {352, 64, 8},     {512, 256, 2},    {832, 256, 4},
    {1024, 512, 2},   {1280, 256, 5},   {1408, 512, 4},   {2552, 512, 5},   {3072, 512, 6},   {4096, 512, 8},
    {5120, 1024, 5},  {6144, 1024, 6},  {7168, 1024, 7},  {8192, 1024, 8}};
constexpr PlanEntry kPlanBF16Unaligned[] = {
    {4, 4, 1},        {8, 4, 2},        {11, 4, 4},       {16, 8, 2},       {22, 8, 4},       {32, 16, 2},
    {48, 16, 4},      {64, 32, 2},      {104, 32, 4},     {128, 64, 2},     {256, 64, 4},     {320, 128, 4},
    {512, 64, 8},     {640, 128, 8},    {1016, 256, 4},   {1272, 256, 5},   {2040, 256, 8},   {2552, 512, 5},
    {3064, 512, 6},   {4096, 512, 8},   {5112, 1024, 5},  {6136, 1024, 6},  {7160, 1024, 7},  {8192, 1024, 8}};

const ResidentShape* find_shape(int lpr, int vpl, int dtype) {
    const int bf = dtype == OS_BF16 ? 1 : 0;
    for (int i = 0; i < kNumResident; ++i)
        if (kResident[i].lpr == lpr && kResident[i].vpl == vpl && kResident[i].fn[bf][0] != nullptr)
            return &kResident[i];
    return nullptr;
}

int64_t vectors_needed(int64_t cols, int dtype) {
    const int64_t vec = 16 / elt_size(dtype);
    return (cols + vec - 1) / vec;
}

// 16-byte slots a row may span: its vectors, or, when row starts are not
// 16-byte aligned, the 16-byte blocks it overlaps (up to VEC - 1 elements
// more at its front).
int64_t slots_needed(int64_t cols, int dtype, bool al) {
    return vectors_needed(al ? cols : cols + 16 / elt_size(dtype) - 1, dtype);
}

// The grid origin of a register-resident launch: the 128-byte line holding
// each row's first element when a workgroup takes one row and the shape holds
// the row from there (up to 127 bytes more at its front; wavefronts then move
// whole cache lines), else the 16-byte block.
uint32_t resident_grid(int lpr, int vpl, int64_t cols, int dtype, bool al) {
    const int64_t es = elt_size(dtype);
    const int64_t lead = al ? 128 - 16 : 128 - es;  // bytes before the first element, at most
    const bool one_row = lpr > 64;
    return one_row && static_cast<int64_t>(lpr) * vpl * 16 >= lead + cols * es + 15 ? kGrid128 : kGrid16;
}

// Every plan entry names a built shape (for bf16: one built for bf16; read
// through LDS: one with that form) that holds its slots, and the entries grow.
template <size_t N>
constexpr bool plan_ok(const PlanEntry (&t)[N], bool bf16) {
    for (size_t i = 0; i < N; ++i) {
        if (static_cast<int64_t>(t[i].lpr) * t[i].vpl < t[i].max_slots) return false;
        if (i > 0 && t[i].max_slots <= t[i - 1].max_slots) return false;
        bool built = false;
        for (int k = 0; k < kNumResident; ++k)
            built = built || (kResident[k].lpr == t[i].lpr && kResident[k].vpl == t[i].vpl &&
                              kResident[k].fn[bf16 ? 1 : 0][0] != nullptr &&
                              (!t[i].staged || kResident[k].staged[bf16 ? 1 : 0] != nullptr));
        if (!built) return false;
    }
    return true;
}
static_assert(plan_ok(kPlanF32, false) && plan_ok(kPlanF32Unaligned, false), "fp32 plan names an unbuilt shape");
static_assert(plan_ok(kPlanBF16, true) && plan_ok(kPlanBF16Unaligned, true), "bf16 plan names an unbuilt shape");
template <size_t N>
constexpr bool never_staged(const PlanEntry (&t)[N]) {
    for (size_t i = 0; i < N; ++i)
        if (t[i].staged) return false;
    return true;
}
static_assert(never_staged(kPlanF32) && never_staged(kPlanBF16), "aligned rows take direct loads");
template <size_t N>
constexpr int last_slots(const PlanEntry (&t)[N]) {
    return t[N - 1].max_slots;
}
// The tables end at 8192 slots (32768 fp32, 65536 bf16 elements).  Longer
// fp32 rows take the hybrid kernel: 1024 lanes x 16 vectors in registers
// (the 1024 x 16 shape, still built for os_softmax_forward_tuned) measured
// 2-8% slower on 40000-65536 columns than 8 vectors in registers plus the
// hybrid's LDS copy, which also reads such rows once.
static_assert(last_slots(kPlanF32) == 8192 && last_slots(kPlanF32Unaligned) == 8192 &&
                  last_slots(kPlanBF16) == 8192 && last_slots(kPlanBF16Unaligned) == 8192,
              "plans end at 8192 slots; longer rows take the hybrid or streaming kernels");

// The plan entry for rows spanning `slots` 16-byte slots (nullptr past 8192).
const PlanEntry* plan_entry(int64_t slots, int dtype, bool al) {
    const PlanEntry* t;
    int n;
    if (dtype == OS_BF16) {
        t = al ? kPlanBF16 : kPlanBF16Unaligned;
        n = al ? sizeof(kPlanBF16) / sizeof(PlanEntry) : sizeof(kPlanBF16Unaligned) / sizeof(PlanEntry);
    } else {
        t = al ? kPlanF32 : kPlanF32Unaligned;
        n = al ? sizeof(kPlanF32) / sizeof(PlanEntry) : sizeof(kPlanF32Unaligned) / sizeof(PlanEntry);
    }
    for (int i = 0; i < n; ++i)
        if (slots <= t[i].max_slots) return &t[i];
    return nullptr;
}

// The plan's shape for rows of `cols` elements, holding every block they span.
void auto_plan(int64_t cols, int dtype, bool al, int* lpr, int* vpl, bool* staged) {
    const PlanEntry* e = plan_entry(slots_needed(cols, dtype, al), dtype, al);
    *lpr = e != nullptr ? e->lpr : 0;
    *vpl = e != nullptr ? e->vpl : 0;
    *staged = e != nullptr && e->staged;
}

// Streaming kernels: 4 vectors per lane per step; waves per row sized to the
// row (1, 4 or 16), so a short row does not idle most of a workgroup.
constexpr int kStreamU = 4;

int stream_waves(int64_t cols, int dtype) {
    const int64_t need = vectors_needed(cols, dtype);
    if (need <= 64 * kStreamU) return 1;
    if (need <= 4 * 64 * kStreamU) return 4;
    return 16;
}

template <int W>
RowKernel stream_kernel_w(int dtype, bool al) {
    if (dtype == OS_BF16) return al ? k_stream<true, W, kStreamU, true> : k_stream<true, W, kStreamU, false>;
    return al ? k_stream<false, W, kStreamU, true> : k_stream<false, W, kStreamU, false>;
}

RowKernel stream_kernel(int w, int dtype, bool al) {
    if (w == 1) return stream_kernel_w<1>(dtype, al);
    if (w == 4) return stream_kernel_w<4>(dtype, al);
    return stream_kernel_w<16>(dtype, al);
}

template <int W>
SafeKernel safe_kernel_w(int dtype, bool al) {
    if (dtype == OS_BF16) return al ? k_safe3<true, W, kStreamU, true> : k_safe3<true, W, kStreamU, false>;
    return al ? k_safe3<false, W, kStreamU, true> : k_safe3<false, W, kStreamU, false>;
}

SafeKernel safe_kernel(int w, int dtype, bool al) {
    if (w == 1) return safe_kernel_w<1>(dtype, al);
    if (w == 4) return safe_kernel_w<4>(dtype, al);
    return safe_kernel_w<16>(dtype, al);
}

typedef void (*SplitFoldKernel)(const void*, State*, int64_t, int, int);
typedef void (*SplitNormKernel)(const void*, void*, const State*, int64_t, int, int);

template <int W>
SplitFoldKernel split_fold_w(int dtype, bool al) {
    if (dtype == OS_BF16) return al ? k_split_fold<true, W, kStreamU, true> : k_split_fold<true, W, kStreamU, false>;
    return al ? k_split_fold<false, W, kStreamU, true> : k_split_fold<false, W, kStreamU, false>;
}

template <int W>
SplitNormKernel split_norm_w(int dtype, bool al) {
    if (dtype == OS_BF16) return al ? k_split_norm<true, W, kStreamU, true> : k_split_norm<true, W, kStreamU, false>;
    return al ? k_split_norm<false, W, kStreamU, true> : k_split_norm<false, W, kStreamU, false>;
}

// Waves per workgroup for a slice of `vecs` 16-byte vectors: the most waves
// whose one tile (waves * 64 lanes * kStreamU vectors) the slice fills, so no
// lane idles through a partly filled tile.
int slice_waves(int64_t vecs) {
    if (vecs >= 16 * 64 * kStreamU) return 16;
    if (vecs >= 8 * 64 * kStreamU) return 8;
    if (vecs >= 4 * 64 * kStreamU) return 4;
    return 1;
}

// A launch may hold at most 2^32 - 1 threads in total; stay below 2^31.
int grid_for(int64_t groups, int block, int requested) {
    const int64_t max_grid = (int64_t(1) << 31) / block;
    int64_t g = requested > 0 ? requested : max_grid;
    if (g > max_grid) g = max_grid;
    if (g > groups) g = groups;
    return static_cast<int>(g);
}

// Rows past the register-resident plans: on rows of up to this many columns
// the hybrid kernel keeps the row's first 1024 x VPL vectors in registers
// (VPL = 7 for bf16; 8, 12 or 16 for fp32 by row length) and the next 4
// streamed tiles (128 KiB) in LDS, and streams the rest twice (measured
// 15-30% faster than streaming the whole row twice up to 262144 columns; no
// better on longer rows, where the on-chip share is small).  bf16 keeps 7
// vectors per lane: with 8 the registers left for the streamed tiles were
// measured 2-4% slower.
constexpr int64_t kHybridMaxCols = 4 * 65536;

// The register-resident shape os_softmax_forward takes for these rows
// (lpr = 0: longer rows, hybrid or streaming), and whether it reads them
// through LDS (*staged).  Rows that are not 16-byte aligned may span one more
// 16-byte block than their length needs (127 bf16 elements: 16 blocks of
// their own, 17 spanned).  Read through LDS, such a row needs only the slots
// of its length, so where the unaligned plan's entry for that length is a
// smaller multi-row shape (at most 128 slots), the row takes it, staged.
// Measured on MI355X on rows one element short of a whole number of blocks
// (4-128 blocks): 1.1-1.2x faster than the shape holding the spanned blocks
// (127 bf16 columns 185 us against 213 us, 15 fp32 columns 173 us against
// 190 us, per ~0.5 GiB); larger staged shapes measured slower than the
// direct shape (bf16 64 x 8 through LDS: 1.7x slower on 4095 columns).
void plan_for(int64_t cols, int dtype, bool al, int* lpr, int* vpl, bool* staged) {
    auto_plan(cols, dtype, al, lpr, vpl, staged);
    if (al || *lpr == 0) return;
    const PlanEntry* s = plan_entry(slots_needed(cols, dtype, true), dtype, false);
    const int64_t cap = static_cast<int64_t>(s->lpr) * s->vpl;
    if (s->lpr <= 64 && cap <= 128 && cap < static_cast<int64_t>(*lpr) * *vpl) {
        *lpr = s->lpr;
        *vpl = s->vpl;
        *staged = true;
    }
}

void plan_rows(const void* in, const void* out, int64_t cols, int dtype, int* lpr, int* vpl, bool* staged) {
    plan_for(cols, dtype, vector_ok(in, out, cols, dtype), lpr, vpl, staged);
}

RowKernel hybrid_kernel(int64_t cols, int dtype, bool al) {
    if (dtype == OS_BF16) return al ? k_hybrid<true, 7, 2, true, 4> : k_hybrid<true, 7, 2, false, 4>;
    // fp32: the register part grows with the row (measured best: 8 vectors
    // per lane up to 65536 columns, all of it on chip with the LDS copy; 12 up
    // to 110000; 16 beyond, where 12 and 16 measured within 1% on 128256 and
    // 16 re-reads less).  Unaligned rows keep 12 beyond 110000: their 16-vector
    // form spills 2 VGPRs, and 12 measured 0.4-3.7% faster on 5 of 6 lengths
    // from 110001 to 262143 columns (2.8% slower at 400 x 150001).
    if (cols <= 65536) return al ? k_hybrid<false, 8, 2, true, 4> : k_hybrid<false, 8, 2, false, 4>;
    if (cols <= 110000 || !al) return al ? k_hybrid<false, 12, 2, true, 4> : k_hybrid<false, 12, 2, false, 4>;
    return k_hybrid<false, 16, 2, true, 4>;
}

int run_rows(const char* fn, const void* in, void* out, RowStats stats, int64_t rows, int64_t cols, int dtype,
             int lpr, int vpl, int grid_req, bool allow_hybrid, bool staged, void* stream) {
    // Shape checks first: no HIP call happens before every argument is known good.
    const bool al = vector_ok(in, out, cols, dtype);
    const ResidentShape* shape = nullptr;
    if (lpr != 0) {
        shape = find_shape(lpr, vpl, dtype);
        if (shape == nullptr)
            return fail(OS_EUNSUPPORTED, "%s: no kernel built for lanes_per_row=%d vecs_per_lane=%d", fn, lpr,
                        vpl);
        if (staged ? (lpr > 64 || shape->staged[dtype == OS_BF16 ? 1 : 0] == nullptr ||
                      static_cast<int64_t>(lpr) * vpl < slots_needed(cols, dtype, true))
                   : static_cast<int64_t>(lpr) * vpl < slots_needed(cols, dtype, al))
            return fail(OS_EINVAL,
                        "%s: lanes_per_row=%d x vecs_per_lane=%d cannot hold %lld columns%s", fn, lpr, vpl,
                        (long long)cols, al ? "" : " (rows not 16-byte aligned span one more 16-byte block)");
    }
    const int bf = dtype == OS_BF16 ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (shape == nullptr) {
        if (allow_hybrid && cols <= kHybridMaxCols) {
            const RowKernel k = hybrid_kernel(cols, dtype, al);
            hipLaunchKernelGGL(k, dim3(grid_for(rows, 1024, grid_req)), dim3(1024), 0, st, in, out, stats, rows,
                               static_cast<int>(cols), kGrid128);
            return launched(fn);
        }
        const int w = stream_waves(cols, dtype);
        const int block = w * 64;
        const int grid = grid_for(rows, block, grid_req);
        hipLaunchKernelGGL(stream_kernel(w, dtype, al), dim3(grid), dim3(block), 0, st, in, out, stats,
                           rows, static_cast<int>(cols), kGrid128);
        return launched(fn);
    }
    const int block = lpr <= 64 ? 256 : lpr;
    const int rpb = block / lpr;
    const int64_t groups = (rows + rpb - 1) / rpb;
    const int grid = grid_for(groups, block, grid_req);
    RowKernel k = staged ? shape->staged[bf] : shape->fn[bf][al ? 1 : 0];
    if (!staged && al && bf == 0 && shape->dense != nullptr && grid_req == 0 && groups <= dense_rows(block))
        k = shape->dense;
    hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, st, in, out, stats, rows, static_cast<int>(cols),
                       staged ? kGrid16 : resident_grid(lpr, vpl, cols, dtype, al));
    return launched(fn);
}

}  // namespace

namespace {

// Workgroups of the read reference (8 per CU; on a 131 MB read this pattern
// measured fastest of the tile and row patterns tried, cold and warm).
constexpr int64_t kReadGrid = 2048;

// The forward with one workgroup (group) per row: the plan os_softmax_forward uses.
int forward_unsplit(const char* fn, const void* in, void* out, int64_t rows, int64_t cols, int dtype, void* stream) {
    int lpr = 0, vpl = 0;
    bool staged = false;
    plan_rows(in, out, cols, dtype, &lpr, &vpl, &staged);
    return run_rows(fn, in, out, RowStats{}, rows, cols, dtype, lpr, vpl, 0, true, staged, stream);
}

// The split forward's two launches over a checked problem, with rows * splits
// slice states at `states` (device memory, no initialisation needed: the first
// launch writes every state before the second reads any).
int forward_split_launch(const char* fn, const void* in, void* out, int64_t rows, int64_t cols, int dtype, int splits,
                         State* states, void* stream) {
    const bool al = vector_ok(in, out, cols, dtype);
    const int64_t seg_vec = (slots_needed(cols, dtype, al) + splits - 1) / splits;
    const int w = slice_waves(seg_vec);
    const int block = w * 64;
    const int64_t units = rows * splits;
    const int grid = grid_for(units, block, 0);
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    const SplitFoldKernel kf = w == 1   ? split_fold_w<1>(dtype, al)
                               : w == 4 ? split_fold_w<4>(dtype, al)
                               : w == 8 ? split_fold_w<8>(dtype, al)
                                        : split_fold_w<16>(dtype, al);
    const SplitNormKernel kn = w == 1   ? split_norm_w<1>(dtype, al)
                               : w == 4 ? split_norm_w<4>(dtype, al)
                               : w == 8 ? split_norm_w<8>(dtype, al)
                                        : split_norm_w<16>(dtype, al);
    hipLaunchKernelGGL(kf, dim3(grid), dim3(block), 0, st, in, states, rows, static_cast<int>(cols), splits);
    const int rc = launched(fn);
    if (rc != OS_OK) return rc;
    hipLaunchKernelGGL(kn, dim3(grid), dim3(block), 0, st, in, out, states, rows, static_cast<int>(cols), splits);
    return launched(fn);
}

// The baselines over global memory: safe softmax in three passes (naive = 0)
// or the unshifted softmax in two (naive = 1), with the lanes-per-row geometry
// the forward picks when the rows fit it, streaming otherwise.
int baseline_forward(const char* fn, const void* in, void* out, int64_t rows, int64_t cols, int dtype, int naive,
                     void* stream) {
    int rc = check_problem(fn, in, out, true, rows, cols, dtype);
    if (rc == 1) return ok();
    if (rc != OS_OK) return rc;
    const bool al = vector_ok(in, out, cols, dtype);
    const int bf = dtype == OS_BF16 ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the safe kernels load directly: every unaligned plan shape, read
    // through LDS by the forward or not, holds the blocks its rows span
    int lpr = 0, vpl = 0;
    bool staged = false;
    auto_plan(cols, dtype, al, &lpr, &vpl, &staged);
    (void)hipGetLastError();
    if (lpr != 0) {
        // rows that fit the register-resident geometry: same lanes and
        // vectors as the forward, every pass over global memory
        const ResidentShape* shape = find_shape(lpr, vpl, dtype);
        const int block = lpr <= 64 ? 256 : lpr;
        const int rpb = block / lpr;
        const int grid = grid_for((rows + rpb - 1) / rpb, block, 0);
        hipLaunchKernelGGL(shape->safe[bf][al ? 1 : 0], dim3(grid), dim3(block), 0, st, in, out, rows,
                           static_cast<int>(cols), resident_grid(lpr, vpl, cols, dtype, al), naive);
    } else {
        const int w = stream_waves(cols, dtype);
        const int block = w * 64;
        const int grid = grid_for(rows, block, 0);
        hipLaunchKernelGGL(safe_kernel(w, dtype, al), dim3(grid), dim3(block), 0, st, in, out, rows,
                           static_cast<int>(cols), kGrid128, naive);
    }
    return launched(fn);
}

// Scratch of os_softmax_forward_split_noalloc: a file-scope device array, so
// that call never allocates.  Each GPU the library runs on holds its own copy
// (OS_STATIC_SCRATCH_BYTES) until the process ends.  In host code `scratch`
// names a host-side stand-in, not device memory: its device address comes from
// hipGetSymbolAddress, looked up once per device (with that device current)
// and kept in g_scratch_addr.
__device__ __align__(256) unsigned char scratch[OS_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The device address of the current device's `scratch`, or an error.
int static_scratch(const char* fn, void** addr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(OS_ELAUNCH, "%s: hipGetDevice failed: %s", fn, hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(OS_ELAUNCH, "%s: device %d outside [0, %d)", fn, dev, kMaxDevices);
    void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_addr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr)
                return fail(OS_ELAUNCH, "%s: hipGetSymbolAddress(scratch) on device %d failed: %s", fn, dev,
                            hipGetErrorString(e));
            g_scratch_addr[dev].store(p, std::memory_order_release);
        }
    }
    *addr = p;
    return OS_OK;
}

}  // namespace

extern "C" {

int os_version(void) { return kVersion; }

const char* os_last_error(void) { return g_error; }

int os_forward_plan(int64_t cols, int dtype, int* lanes_per_row, int* vecs_per_lane) {
    if (dtype != OS_F32 && dtype != OS_BF16) return fail(OS_EINVAL, "os_forward_plan: unknown dtype %d", dtype);
    if (cols < 0 || cols > OS_MAX_COLS) return fail(OS_EINVAL, "os_forward_plan: cols %lld out of range", (long long)cols);
    if (lanes_per_row == nullptr || vecs_per_lane == nullptr)
        return fail(OS_EINVAL, "os_forward_plan: NULL output pointer");
    // rows of a 16-byte aligned array: aligned when the row bytes are a multiple of 16
    bool staged = false;
    plan_for(cols, dtype, (cols * elt_size(dtype)) % 16 == 0, lanes_per_row, vecs_per_lane, &staged);
    return ok();
}

int os_softmax_forward(const void* in, void* out, int64_t rows, int64_t cols, int dtype, void* stream) {
    const char* fn = "os_softmax_forward";
    int rc = check_problem(fn, in, out, true, rows, cols, dtype);
    if (rc == 1) return ok();
    if (rc != OS_OK) return rc;
    int lpr = 0, vpl = 0;
    bool staged = false;
    plan_rows(in, out, cols, dtype, &lpr, &vpl, &staged);
    return run_rows(fn, in, out, RowStats{}, rows, cols, dtype, lpr, vpl, 0, true, staged, stream);
}

int os_softmax_forward_tuned(const void* in, void* out, int64_t rows, int64_t cols, int dtype, int lanes_per_row,
                             int vecs_per_lane, int grid_blocks, void* stream) {
    const char* fn = "os_softmax_forward_tuned";
    int rc = check_problem(fn, in, out, true, rows, cols, dtype);
    if (rc != OS_OK && rc != 1) return rc;
    if (lanes_per_row < 0 || grid_blocks < 0)
        return fail(OS_EINVAL, "%s: lanes_per_row and grid_blocks must be >= 0", fn);
    if (lanes_per_row != 0 && find_shape(lanes_per_row, vecs_per_lane, dtype) == nullptr)
        return fail(OS_EUNSUPPORTED, "%s: no kernel built for lanes_per_row=%d vecs_per_lane=%d", fn, lanes_per_row,
                    vecs_per_lane);
    if (rc == 1) return ok();
    return run_rows(fn, in, out, RowStats{}, rows, cols, dtype, lanes_per_row, vecs_per_lane, grid_blocks, false, false,
                    stream);
}

int os_softmax_stats(const void* in, float* m, float* d, int64_t rows, int64_t cols, int dtype, void* stream) {
    const char* fn = "os_softmax_stats";
    int rc = check_problem(fn, in, nullptr, false, rows, cols, dtype);
    if (rc != OS_OK && rc != 1) return rc;
    if (rows == 0) return ok();
    if (m == nullptr || d == nullptr) return fail(OS_EINVAL, "%s: m and d must not be NULL", fn);
    if (!aligned(m, 4) || !aligned(d, 4)) return fail(OS_EINVAL, "%s: m and d must be 4-byte aligned", fn);
    // cols == 0: every row is empty and gets the identity state; the input is never read.
    int lpr = 0, vpl = 0;
    bool staged = false;
    plan_rows(in, nullptr, cols, dtype, &lpr, &vpl, &staged);
    return run_rows(fn, cols == 0 ? nullptr : in, nullptr, RowStats{m, d, nullptr}, rows, cols, dtype, lpr, vpl, 0,
                    true, staged, stream);
}

int os_softmax_forward_lse(const void* in, void* out, float* lse, int64_t rows, int64_t cols, int dtype,
                           void* stream) {
    const char* fn = "os_softmax_forward_lse";
    int rc = check_problem(fn, in, out, false, rows, cols, dtype);
    if (rc != OS_OK && rc != 1) return rc;
    if (rows == 0) return ok();
    if (lse == nullptr) return fail(OS_EINVAL, "%s: lse must not be NULL", fn);
    if (!aligned(lse, 4)) return fail(OS_EINVAL, "%s: lse must be 4-byte aligned", fn);
    // cols == 0: every row is empty, L = -inf; neither x nor y is touched.
    int lpr = 0, vpl = 0;
    bool staged = false;
    plan_rows(in, out, cols, dtype, &lpr, &vpl, &staged);
    return run_rows(fn, cols == 0 ? nullptr : in, cols == 0 ? nullptr : out, RowStats{nullptr, nullptr, lse}, rows,
                    cols, dtype, lpr, vpl, 0, true, staged, stream);
}

int64_t os_softmax_forward_workspace_bytes(int64_t rows, int splits) {
    if (rows < 0 || splits < 1 || splits > OS_FWD_MAX_SPLITS ||
        !workspace_fits(rows, splits * static_cast<int64_t>(sizeof(State)))) {
        fail(OS_EINVAL, "os_softmax_forward_workspace_bytes: bad rows or splits");
        return OS_EINVAL;
    }
    ok();
    return splits == 1 ? 0 : rows * splits * static_cast<int64_t>(sizeof(State));
}

int os_forward_split_plan(int64_t rows, int64_t cols, int dtype) {
    if (rows <= 0 || cols <= 0 || cols > OS_MAX_COLS || (dtype != OS_F32 && dtype != OS_BF16)) return 1;
    // Rows of up to 65536 elements are read once (registers, or registers
    // and LDS) and are not split (the second launch and read cost more than
    // idle CUs on every batch measured).  Longer rows are split into the most
    // slices that keep the batch at <= 256 workgroups (one per CU) and every
    // slice >= 1024 vectors (16 KB) (measured on MI355X over 1..256 rows of
    // 128256 to 2^24 columns, fp32 and bf16).
    if (cols <= 65536) return 1;
    const int64_t vecs = vectors_needed(cols, dtype);
    int S = 1;
    while (S < OS_FWD_MAX_SPLITS && rows * S * 2 <= 256 && vecs / (S * 2) >= 1024) S *= 2;
    return S;
}

int os_softmax_forward_split(const void* in, void* out, int64_t rows, int64_t cols, int dtype, int splits,
                             void* workspace, int64_t workspace_bytes, void* stream) {
    const char* fn = "os_softmax_forward_split";
    if (splits < 1 || splits > OS_FWD_MAX_SPLITS)
        return fail(OS_EINVAL, "%s: splits=%d outside [1, %d]", fn, splits, OS_FWD_MAX_SPLITS);
    int rc = check_problem(fn, in, out, true, rows, cols, dtype);
    if (rc == 1) return ok();
    if (rc != OS_OK) return rc;
    if (splits == 1) return forward_unsplit(fn, in, out, rows, cols, dtype, stream);
    if (!workspace_fits(rows, splits * static_cast<int64_t>(sizeof(State))))
        return fail(OS_EINVAL, "%s: rows * splits overflows the workspace size", fn);
    const int64_t need = rows * splits * static_cast<int64_t>(sizeof(State));
    if (workspace == nullptr) return fail(OS_EINVAL, "%s: splits > 1 needs a workspace", fn);
    if (!aligned(workspace, 8)) return fail(OS_EINVAL, "%s: workspace must be 8-byte aligned", fn);
    if (workspace_bytes < need)
        return fail(OS_EINVAL, "%s: workspace has %lld bytes, needs %lld", fn, (long long)workspace_bytes,
                    (long long)need);
    return forward_split_launch(fn, in, out, rows, cols, dtype, splits, static_cast<State*>(workspace), stream);
}

int os_softmax_forward_split_noalloc(const void* in, void* out, int64_t rows, int64_t cols, int dtype, int splits,
                                     void* stream) {
    const char* fn = "os_softmax_forward_split_noalloc";
    if (splits < 1 || splits > OS_FWD_MAX_SPLITS)
        return fail(OS_EINVAL, "%s: splits=%d outside [1, %d]", fn, splits, OS_FWD_MAX_SPLITS);
    int rc = check_problem(fn, in, out, true, rows, cols, dtype);
    if (rc == 1) return ok();
    if (rc != OS_OK) return rc;
    if (splits == 1) return forward_unsplit(fn, in, out, rows, cols, dtype, stream);
    if (rows > OS_STATIC_SCRATCH_BYTES / (splits * static_cast<int64_t>(sizeof(State))))
        return fail(OS_EINVAL, "%s: rows * splits * %d bytes exceeds the %lld-byte static scratch", fn,
                    (int)sizeof(State), (long long)OS_STATIC_SCRATCH_BYTES);
    State* states = nullptr;
    rc = static_scratch(fn, reinterpret_cast<void**>(&states));
    if (rc != OS_OK) return rc;
    return forward_split_launch(fn, in, out, rows, cols, dtype, splits, states, stream);
}

int safe_softmax_forward(const void* in, void* out, int64_t rows, int64_t cols, int dtype, void* stream) {
    return baseline_forward("safe_softmax_forward", in, out, rows, cols, dtype, 0, stream);
}

int naive_softmax_forward(const void* in, void* out, int64_t rows, int64_t cols, int dtype, void* stream) {
    return baseline_forward("naive_softmax_forward", in, out, rows, cols, dtype, 1, stream);
}

}  // extern "C"

namespace {

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

// Workspace of the split launch: [rows*S] states | [rows*S*K] list entries,
// each part 256-byte aligned.
struct TopkWorkspace {
    int64_t states_off, lists_off, bytes;
};

TopkWorkspace topk_workspace(int64_t rows, int K, int S) {
    TopkWorkspace w;
    w.states_off = 0;
    w.lists_off = align256(rows * S * static_cast<int64_t>(sizeof(State)));
    w.bytes = w.lists_off + rows * S * K * static_cast<int64_t>(sizeof(TopkEntry));
    return w;
}

int check_topk(const char* fn, const void* in, int dtype, const float* probs, const int32_t* idx, int64_t rows,
               int64_t cols, int K) {
    if (dtype != OS_F32 && dtype != OS_BF16) return fail(OS_EINVAL, "%s: unknown dtype %d", fn, dtype);
    if (rows < 0 || cols < 0) return fail(OS_EINVAL, "%s: rows and cols must be >= 0", fn);
    if (cols > OS_MAX_COLS) return fail(OS_EINVAL, "%s: cols %lld exceeds OS_MAX_COLS", fn, (long long)cols);
    if (K < 1 || K > OS_TOPK_KMAX) return fail(OS_EINVAL, "%s: K=%d outside [1, %d]", fn, K, OS_TOPK_KMAX);
    if (rows == 0) return 1;
    if (static_cast<int64_t>(K) > cols) return fail(OS_EINVAL, "%s: K=%d exceeds cols=%lld", fn, K, (long long)cols);
    if (rows > INT64_MAX / cols / 4) return fail(OS_EINVAL, "%s: rows * cols overflows", fn);
    if (in == nullptr || probs == nullptr || idx == nullptr) return fail(OS_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(in, elt_size(dtype)) || !aligned(probs, 4) || !aligned(idx, 4))
        return fail(OS_EINVAL, "%s: input must be aligned to its element size, probs and idx to 4 bytes", fn);
    return OS_OK;
}

typedef void (*TopkKernel)(const void*, float*, int*, int64_t, int, int, int, State*, TopkEntry*, int);

// Vectors per lane per tile: 4 for fp32, 2 for bf16 (16 elements either way).
template <int W, bool BF16>
TopkKernel topk_kernel_t(bool al, bool split) {
    constexpr int U = BF16 ? 2 : 4;
    if (split) return al ? k_topk<BF16, W, U, true, true> : k_topk<BF16, W, U, false, true>;
    return al ? k_topk<BF16, W, U, true, false> : k_topk<BF16, W, U, false, false>;
}

template <int W>
TopkKernel topk_kernel(int dtype, bool al, bool split) {
    return dtype == OS_BF16 ? topk_kernel_t<W, true>(al, split) : topk_kernel_t<W, false>(al, split);
}

// Waves per workgroup for the top-K of `units` rows (or row slices) of
// `seg_cols` columns, from a sweep on MI355X over 64..16384 rows of 512..128256
// columns, K = 1, 8, 32, fp32 and bf16, every width from 1 to 16 timed.
//   - Long rows on few workgroups want 16 waves, to keep enough loads in
//     flight per CU.
//   - Short rows, or many workgroups, want few, since every wave pays for its
//     own threshold and K-list and the workgroup for the final merge.  A large
//     K wants more, so that the lists build in parallel.
//   - The first bound on the K-th value is taken over 64 parts of the
//     workgroup's first tile, so a row should give each of at least 2 K parts
//     some of its 16-byte slots: W <= slots / (2 K).
// Tables by K (<= 8, more), columns (<= 512, 2048, 8192, 32768, longer) and
// workgroups (<= 64, 256, 1024, 4096, more).  The choice is within 6.3% of
// the best width at every swept point, and 0.4% on average.  A fixed width
// was up to 10x off for short rows on many workgroups.
int topk_waves(int64_t units, int64_t seg_cols, int K, int dtype) {
    static const int kWaves[2][5][5] = {
        {
            {4, 4, 2, 1, 1},       // K <= 8: <= 512 columns
            {4, 4, 2, 1, 1},       // <= 2048
            {8, 8, 4, 4, 2},       // <= 8192
            {16, 16, 4, 4, 4},     // <= 32768
            {16, 16, 4, 8, 8},     // longer
        },
        {
            {2, 2, 2, 1, 1},       // K > 8
            {4, 4, 4, 2, 2},
            {8, 8, 4, 4, 4},
            {16, 16, 8, 8, 8},
            {16, 16, 8, 8, 8},
        }};
    const int cb = seg_cols <= 512 ? 0 : seg_cols <= 2048 ? 1 : seg_cols <= 8192 ? 2 : seg_cols <= 32768 ? 3 : 4;
    const int rb = units <= 64 ? 0 : units <= 256 ? 1 : units <= 1024 ? 2 : units <= 4096 ? 3 : 4;
    int W = kWaves[K > 8 ? 1 : 0][cb][rb];
    const int64_t slots = vectors_needed(seg_cols, dtype);
    while (W > 1 && static_cast<int64_t>(W) * 2 * K > slots) W /= 2;
    return W;
}

// Register-resident top-K shapes for short rows (up to 2048 columns): lanes
// per row x 16-byte slots per lane, 32 entries per lane (fp32 8 slots, bf16 4)
// or fewer on the shortest rows, by capacity.
typedef void (*TopkRowsKernel)(const void*, float*, int*, int64_t, int, int);
struct TopkRowsShape {
    int lpr, vpl;
    TopkRowsKernel fn[2][2];  // [K == 1][aligned]
};
// bf16 rows select on packed (key, column) entries (k_topk_rows_bf16) for
// K >= 2: 5-74% faster than k_topk_rows on 65536 x 16 .. 4096 x 2048 at
// K = 2..32 (16384 x 512 K = 32: 14.5 us instead of 23.7; 65536 x 1024 K = 16:
// 68.5 us instead of 94.6).  At K = 1 it measured -3.6% to +1.3% (its
// register form holds more VGPRs), so K = 1 keeps k_topk_rows.
template <bool B, int L, int V, bool AL, bool FEWK>
constexpr TopkRowsKernel topk_rows_fn() {
    if constexpr (B && !FEWK) return k_topk_rows_bf16<L, V, AL, false>;
    else return k_topk_rows<B, L, V, AL, FEWK>;
}
#define ONORM_TOPK_ROWS(B, L, V)                                                                       \
    {                                                                                                  \
        L, V, {                                                                                        \
            {topk_rows_fn<B, L, V, false, false>(), topk_rows_fn<B, L, V, true, false>()},             \
            {topk_rows_fn<B, L, V, false, true>(), topk_rows_fn<B, L, V, true, true>()}                \
        }                                                                                              \
    }
const TopkRowsShape kTopkRowsF32[] = {
    ONORM_TOPK_ROWS(false, 4, 1),  ONORM_TOPK_ROWS(false, 4, 2),  ONORM_TOPK_ROWS(false, 4, 4),
    ONORM_TOPK_ROWS(false, 4, 8),  ONORM_TOPK_ROWS(false, 8, 8),  ONORM_TOPK_ROWS(false, 16, 8),
    ONORM_TOPK_ROWS(false, 32, 8), ONORM_TOPK_ROWS(false, 64, 8)};
const TopkRowsShape kTopkRowsBF16[] = {
    ONORM_TOPK_ROWS(true, 4, 1),  ONORM_TOPK_ROWS(true, 4, 2),  ONORM_TOPK_ROWS(true, 4, 4),
    ONORM_TOPK_ROWS(true, 8, 4),  ONORM_TOPK_ROWS(true, 16, 4), ONORM_TOPK_ROWS(true, 32, 4), ONORM_TOPK_ROWS(true, 64, 4)};
#undef ONORM_TOPK_ROWS
// 64 entries per lane (K >= 2 only): half the lanes per row of the shapes
// above, so each of the K rounds serves twice the rows per wavefront with one
// butterfly step fewer, at 64 KiB of LDS keys per workgroup (2 waves per SIMD).
#define ONORM_TOPK_WIDE(B, L, V)                                                     \
    {                                                                                \
        L, V, {                                                                      \
            {topk_rows_fn<B, L, V, false, false>(), topk_rows_fn<B, L, V, true, false>()}, \
            {nullptr, nullptr}                                                       \
        }                                                                            \
    }
// (fp32 rows of <= 256 columns keep 8 lanes: 4 x 16 ran 14% slower at
// 40000 x 200 for K = 32 and gained 2% at 65536 x 256)
const TopkRowsShape kTopkWideF32[] = {ONORM_TOPK_WIDE(false, 8, 16), ONORM_TOPK_WIDE(false, 16, 16)};
const TopkRowsShape kTopkWideBF16[] = {ONORM_TOPK_WIDE(true, 4, 8), ONORM_TOPK_WIDE(true, 8, 8),
                                       ONORM_TOPK_WIDE(true, 16, 8)};
#undef ONORM_TOPK_WIDE

// The short-row shape for these rows, or nullptr when they are too long: the
// fewest lanes per row that hold it (measured best on rows of 128..512
// columns against 2..16 times the lanes).  Batches with many rounds (K >= 32)
// take the 64-entry shape when it has fewer lanes and still gives each SIMD
// two waves (rows x lanes >= 2 x 256 CUs x 256 lanes); measured on MI355X over
// 256..1024 columns and 4096..65536 rows, those cases ran 2..20% faster
// (16384 x 512 fp32 K = 32: 24.5 us instead of 28.8 us; bf16 on packed
// entries 14.3 us instead of 17.1 us), and with one wave per SIMD
// (16384 x 256) they ran up to 28% slower.  At K = 16 bf16 rows on packed
// entries measured -7% to +12%, so both dtypes start at K = 32.  Through the tiled
// kernel before this rule, 65536 x 1024 for K = 32 took 242 us (fp32) and
// 215 us (bf16); now 169 us and 155 us.
const TopkRowsShape* topk_rows_shape(int64_t rows, int64_t cols, int K, int dtype, bool al) {
    const int64_t need = slots_needed(cols, dtype, al);
    const bool bf = dtype == OS_BF16;
    const TopkRowsShape* t = bf ? kTopkRowsBF16 : kTopkRowsF32;
    const int n = bf ? sizeof(kTopkRowsBF16) / sizeof(kTopkRowsBF16[0]) : sizeof(kTopkRowsF32) / sizeof(kTopkRowsF32[0]);
    const TopkRowsShape* best = nullptr;
    for (int i = 0; i < n && best == nullptr; ++i)
        if (static_cast<int64_t>(t[i].lpr) * t[i].vpl >= need) best = &t[i];
    if (best == nullptr || K < 32) return best;
    const TopkRowsShape* w = bf ? kTopkWideBF16 : kTopkWideF32;
    const int nw = bf ? sizeof(kTopkWideBF16) / sizeof(kTopkWideBF16[0]) : sizeof(kTopkWideF32) / sizeof(kTopkWideF32[0]);
    for (int i = 0; i < nw; ++i)
        if (static_cast<int64_t>(w[i].lpr) * w[i].vpl >= need)
            return w[i].lpr < best->lpr && rows * w[i].lpr >= 2 * 256 * 256 ? &w[i] : best;
    return best;
}

// Whether the short-row kernel serves this batch (unsplit rows only).  Each
// of its rows is one dependent chain of K rounds, so it wins on short rows,
// on many rows (where the tiled kernel pays its per-workgroup cost per row)
// and for small K; on a few wide rows the tiled kernel's waves share the
// selection instead.  Largest K it serves, by row length (<= 16, 64, 128,
// 256, 512, 1024, 2048 columns; longer rows never) and batch (< 2048,
// < 4096, < 8192, more rows), measured on MI355X against the tiled kernel
// over 64..65536 rows, K = 1..32, both dtypes: where it is used it was as
// fast or faster (up to 23x at 65536 rows of 16, 4.6x at 65536 x 256 for
// K = 8, 1.2-1.6x on rows of 1500-2048 for K <= 2, 1.4x at 65536 x 1024 for
// K = 32), and where it is not it was slower.
// bf16 rows select on packed entries, which made each round about half as
// costly; the same comparison then favoured this kernel far more often (e.g.
// 3000 x 256 at K = 8: 4.8 us against 8.5; 65536 x 1024 at K = 32: 101 us
// against 215), and the tiled kernel kept only small batches of long rows at
// large K (64 x 1024 at K = 32: 8.0 us against 10.6) and K = 32 on rows of
// 1025-2048 columns.
bool use_topk_rows(int64_t rows, int64_t cols, int K, int dtype, bool al) {
    static const int kMaxKBF16[7][4] = {
        {32, 32, 32, 32},  // <= 16 columns
        {32, 32, 32, 32},  // <= 64
        {32, 32, 32, 32},  // <= 128
        {32, 32, 32, 32},  // <= 256
        {16, 32, 32, 32},  // <= 512
        {8, 32, 32, 32},   // <= 1024
        {4, 32, 16, 16},   // <= 2048
    };
    // fp32, re-measured after the butterfly became two integer reductions
    // (64..65536 rows x 64..2048 columns, K = 1..32; a limit holds where the
    // rows kernel was within 2% or faster at the measured batches on both
    // sides of the bucket's lower edge)
    static const int kMaxK[7][4] = {
        {32, 32, 32, 32},  // <= 16 columns
        {32, 32, 32, 32},  // <= 64
        {8, 32, 32, 32},   // <= 128
        {4, 8, 16, 32},    // <= 256
        {2, 8, 16, 32},    // <= 512
        {2, 8, 16, 32},    // <= 1024
        {2, 8, 8, 4},      // <= 2048
    };
    if (cols > 2048 || topk_rows_shape(rows, cols, K, dtype, al) == nullptr) return false;
    const int cb = cols <= 16    ? 0
                   : cols <= 64  ? 1
                   : cols <= 128 ? 2
                   : cols <= 256 ? 3
                   : cols <= 512 ? 4
                   : cols <= 1024 ? 5
                                  : 6;
    const int rb = rows < 2048 ? 0 : rows < 4096 ? 1 : rows < 8192 ? 2 : 3;
    return K <= (dtype == OS_BF16 ? kMaxKBF16[cb][rb] : kMaxK[cb][rb]);
}

int launch_topk(const char* fn, const void* in, int dtype, float* probs, int32_t* idx, int64_t rows, int64_t cols,
                int K, int S, void* workspace, void* stream, int select = 0) {
    const bool al = aligned(in, 16) && ((cols * elt_size(dtype)) % 16) == 0;
    if (S == 1 && !select && use_topk_rows(rows, cols, K, dtype, al)) {
        const TopkRowsShape* sh = topk_rows_shape(rows, cols, K, dtype, al);
        const int rpb = 256 / sh->lpr;
        (void)hipGetLastError();
        // K = 1 without LDS measured up to 8% faster; for K = 2 the register
        // rescan cost up to 13% against the LDS group refresh
        hipLaunchKernelGGL(sh->fn[K == 1 ? 1 : 0][al ? 1 : 0], dim3(grid_for((rows + rpb - 1) / rpb, 256, 0)), dim3(256), 0,
                           static_cast<hipStream_t>(stream), in, probs, idx, rows, static_cast<int>(cols), K);
        return launched(fn);
    }
    const int64_t units = rows * S;
    const int W = topk_waves(units, (cols + S - 1) / S, K, dtype);
    const int block = W * 64;
    const int grid = grid_for(units, block, 0);
    const bool split = S > 1;
    const TopkKernel k = W == 1   ? topk_kernel<1>(dtype, al, split)
                         : W == 2 ? topk_kernel<2>(dtype, al, split)
                         : W == 4 ? topk_kernel<4>(dtype, al, split)
                         : W == 8 ? topk_kernel<8>(dtype, al, split)
                                  : topk_kernel<16>(dtype, al, split);
    State* states = nullptr;
    TopkEntry* lists = nullptr;
    if (S > 1) {
        const TopkWorkspace w = topk_workspace(rows, K, S);
        char* base = static_cast<char*>(workspace);
        states = reinterpret_cast<State*>(base + w.states_off);
        lists = reinterpret_cast<TopkEntry*>(base + w.lists_off);
    }
    hipStream_t st = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k, dim3(grid), dim3(block), 0, st, in, probs, idx, rows, static_cast<int>(cols), K, S,
                       states, lists, select);
    if (S > 1) {
        const int rc = launched(fn);
        if (rc != OS_OK) return rc;
        const int mgrid = grid_for((rows + 3) / 4, 256, 0);
        hipLaunchKernelGGL(k_topk_merge, dim3(mgrid), dim3(256), 0, st, probs, idx, rows, K, S, states, lists);
    }
    return launched(fn);
}

int topk_split_common(const char* fn, const void* in, int dtype, float* probs, int32_t* idx, int64_t rows,
                      int64_t cols, int K, int splits, void* workspace, int64_t workspace_bytes, void* stream) {
    if (splits < 1 || splits > OS_TOPK_MAX_SPLITS)
        return fail(OS_EINVAL, "%s: splits=%d outside [1, %d]", fn, splits, OS_TOPK_MAX_SPLITS);
    const int rc = check_topk(fn, in, dtype, probs, idx, rows, cols, K);
    if (rc == 1) return ok();
    if (rc != OS_OK) return rc;
    if (splits > 1) {
        if (!workspace_fits(rows, splits * static_cast<int64_t>(sizeof(State) + K * sizeof(TopkEntry)) + 512))
            return fail(OS_EINVAL, "%s: rows * splits overflows the workspace size", fn);
        if (workspace == nullptr) return fail(OS_EINVAL, "%s: workspace is NULL", fn);
        if (!aligned(workspace, 256)) return fail(OS_EINVAL, "%s: workspace must be 256-byte aligned", fn);
        const int64_t need = topk_workspace(rows, K, splits).bytes;
        if (workspace_bytes < need)
            return fail(OS_EINVAL, "%s: workspace has %lld bytes, needs %lld", fn, (long long)workspace_bytes,
                        (long long)need);
    }
    return launch_topk(fn, in, dtype, probs, idx, rows, cols, K, splits, workspace, stream);
}

}  // namespace

extern "C" {

int os_softmax_topk(const float* in, float* probs, int32_t* idx, int64_t rows, int64_t cols, int K, void* stream) {
    const char* fn = "os_softmax_topk";
    const int rc = check_topk(fn, in, OS_F32, probs, idx, rows, cols, K);
    if (rc == 1) return ok();
    if (rc != OS_OK) return rc;
    return launch_topk(fn, in, OS_F32, probs, idx, rows, cols, K, 1, nullptr, stream);
}

int64_t os_softmax_topk_workspace_bytes(int64_t rows, int K, int splits) {
    if (rows < 0 || K < 1 || K > OS_TOPK_KMAX || splits < 1 || splits > OS_TOPK_MAX_SPLITS ||
        !workspace_fits(rows, splits * static_cast<int64_t>(sizeof(State) + K * sizeof(TopkEntry)) + 512)) {
        fail(OS_EINVAL, "os_softmax_topk_workspace_bytes: bad rows, K or splits");
        return OS_EINVAL;
    }
    ok();
    return splits == 1 ? 0 : topk_workspace(rows, K, splits).bytes;
}

int os_topk_plan(int64_t rows, int64_t cols, int K) {
    if (rows <= 0 || cols <= 0 || K < 1) return 1;
    // Splitting pays only for batches far smaller than the CU count, and only
    // for rows long enough that streaming one on a single workgroup outlasts
    // the second (merge) launch.  Measured on MI355X with graph-timed
    // launches:
    //   - 16 and 32 rows x 128256 are best at 8 slices, 64 rows at 4 or 8;
    //   - 128 and 256 rows are best unsplit, or within 2% of it;
    //   - rows of 32000..65536 columns are best unsplit at 32..256 rows
    //     (128 x 65536: 10.1 us unsplit, 13.8 us at 2 slices).
    // So: at most 64 rows, rows of >= 96K columns, at most 256 workgroups and
    // 8 slices, slices of >= 8K columns.
    if (cols < 98304 || rows > 64) return 1;
    int S = 1;
    while (S < 8 && rows * S * 2 <= 256 && cols / (S * 2) >= 8192) S *= 2;
    return S;
}

int os_softmax_topk_split(const float* in, float* probs, int32_t* idx, int64_t rows, int64_t cols, int K, int splits,
                          void* workspace, int64_t workspace_bytes, void* stream) {
    return topk_split_common("os_softmax_topk_split", in, OS_F32, probs, idx, rows, cols, K, splits, workspace,
                             workspace_bytes, stream);
}

int os_softmax_topk_ex(const void* in, int dtype, float* probs, int32_t* idx, int64_t rows, int64_t cols, int K,
                       int splits, void* workspace, int64_t workspace_bytes, void* stream) {
    return topk_split_common("os_softmax_topk_ex", in, dtype, probs, idx, rows, cols, K, splits, workspace,
                             workspace_bytes, stream);
}

int os_topk_select(const void* in, int dtype, float* vals, int32_t* idx, int64_t rows, int64_t cols, int K,
                   void* stream) {
    const char* fn = "os_topk_select";
    const int rc = check_topk(fn, in, dtype, vals, idx, rows, cols, K);
    if (rc == 1) return ok();
    if (rc != OS_OK) return rc;
    return launch_topk(fn, in, dtype, vals, idx, rows, cols, K, 1, nullptr, stream, 1);
}

int os_device_copy(const void* src, void* dst, int64_t bytes, void* stream) {
    const char* fn = "os_device_copy";
    if (bytes < 0 || bytes % 16 != 0) return fail(OS_EINVAL, "%s: bytes must be a non-negative multiple of 16", fn);
    if (bytes == 0) return ok();
    if (src == nullptr || dst == nullptr) return fail(OS_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(OS_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    const char* s = static_cast<const char*>(src);
    const char* d = static_cast<const char*>(dst);
    if (s < d + bytes && d < s + bytes) return fail(OS_EINVAL, "%s: source and destination overlap", fn);
    const int64_t tiles = (bytes + 4095) / 4096;
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_copy, dim3(grid_for(tiles, 256, 0)), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const char*>(src), static_cast<char*>(dst), bytes);
    return launched(fn);
}

int os_bench_exp(float* out, int64_t workgroups, int iters, int chains, void* stream) {
    const char* fn = "os_bench_exp";
    if (chains != 1 && chains != 8) return fail(OS_EINVAL, "%s: chains must be 1 or 8", fn);
    if (workgroups < 1 || workgroups > (int64_t(1) << 20) || iters < 1)
        return fail(OS_EINVAL, "%s: workgroups must be in [1, 2^20] and iters >= 1", fn);
    if (out == nullptr || !aligned(out, 4)) return fail(OS_EINVAL, "%s: out must be a 4-byte aligned pointer", fn);
    (void)hipGetLastError();
    hipLaunchKernelGGL(chains == 1 ? k_exp_rate<1> : k_exp_rate<8>, dim3(static_cast<uint32_t>(workgroups)), dim3(256),
                       0, static_cast<hipStream_t>(stream), out, iters);
    return launched(fn);
}

int os_attention_forward(const void* q, const void* k, const void* v, void* o, float* lse, int64_t heads, int64_t nq,
                         int64_t nk, int head_dim, float scale, int causal, void* stream) {
    const char* fn = "os_attention_forward";
    if (head_dim != kAttnD) return fail(OS_EINVAL, "%s: head_dim %d is not supported (128 only)", fn, head_dim);
    if (heads < 0 || nq < 0 || nk < 0) return fail(OS_EINVAL, "%s: heads, nq and nk must be >= 0", fn);
    if (heads == 0 || nq == 0) return ok();
    if (nk < 1) return fail(OS_EINVAL, "%s: nk must be >= 1 when there are query rows", fn);
    if (nq > OS_ATTN_MAX_SEQ || nk > OS_ATTN_MAX_SEQ)
        return fail(OS_EINVAL, "%s: nq and nk must be <= %lld", fn, (long long)OS_ATTN_MAX_SEQ);
    if (causal && nq != nk) return fail(OS_EINVAL, "%s: the causal mask needs nq == nk", fn);
    if (!(scale > 0.0f) || !(scale < INFINITY)) return fail(OS_EINVAL, "%s: scale must be finite and > 0", fn);
    const int64_t nqb = (nq + kAttnBr - 1) / kAttnBr;
    if (heads > INT64_MAX / (nq > nk ? nq : nk) / kAttnD / 2 || heads > INT64_MAX / nqb)
        return fail(OS_EINVAL, "%s: heads * rows * head_dim overflows", fn);
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr) return fail(OS_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
        return fail(OS_EINVAL, "%s: q, k, v, o must be 16-byte aligned and lse 4-byte aligned", fn);
    const int64_t units = heads * nqb;
    const int grid = grid_for(units, kAttnWaves * 64, 0);
    (void)hipGetLastError();
    hipLaunchKernelGGL(causal ? k_attn_fwd<true> : k_attn_fwd<false>, dim3(grid), dim3(kAttnWaves * 64), 0,
                       static_cast<hipStream_t>(stream), static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse,
                       heads, static_cast<int>(nq), static_cast<int>(nk), scale);
    return launched(fn);
}

int os_device_read(const void* src, int64_t bytes, float* sink, int64_t sink_floats, void* stream) {
    const char* fn = "os_device_read";
    if (bytes < 0 || bytes % 16 != 0) return fail(OS_EINVAL, "%s: bytes must be a non-negative multiple of 16", fn);
    if (bytes == 0) return ok();
    if (src == nullptr || sink == nullptr) return fail(OS_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(src, 16) || !aligned(sink, 4)) return fail(OS_EINVAL, "%s: src must be 16-byte and sink 4-byte aligned", fn);
    const int64_t tiles = (bytes + 4095) / 4096;
    const int grid = static_cast<int>(tiles < kReadGrid ? tiles : kReadGrid);
    if (sink_floats < static_cast<int64_t>(grid) * 4)
        return fail(OS_EINVAL, "%s: sink holds %lld floats, needs %lld", fn, (long long)sink_floats, (long long)grid * 4);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_read, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream), static_cast<const char*>(src),
                       bytes, sink);
    return launched(fn);
}

int os_device_copy_rows(const void* src, void* dst, int64_t rows, int64_t row_bytes, void* stream) {
    const char* fn = "os_device_copy_rows";
    if (rows < 0 || row_bytes < 0 || row_bytes % 16 != 0 || row_bytes > 131072)
        return fail(OS_EINVAL, "%s: row_bytes must be a multiple of 16 in [0, 131072]", fn);
    if (rows == 0 || row_bytes == 0) return ok();
    if (rows > INT64_MAX / row_bytes) return fail(OS_EINVAL, "%s: rows * row_bytes overflows", fn);
    if (src == nullptr || dst == nullptr) return fail(OS_EINVAL, "%s: NULL pointer", fn);
    if (!aligned(src, 16) || !aligned(dst, 16)) return fail(OS_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    const int64_t bytes = rows * row_bytes;
    const char* s = static_cast<const char*>(src);
    const char* d = static_cast<const char*>(dst);
    if (s < d + bytes && d < s + bytes) return fail(OS_EINVAL, "%s: source and destination overlap", fn);
    (void)hipGetLastError();
    hipLaunchKernelGGL(k_copy_rows, dim3(grid_for(rows, 1024, 0)), dim3(1024), 0, static_cast<hipStream_t>(stream), s,
                       static_cast<char*>(dst), rows, static_cast<uint32_t>(row_bytes));
    return launched(fn);
}

}  // extern "C"

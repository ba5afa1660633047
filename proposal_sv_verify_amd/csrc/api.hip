// api.hip -- host side of libspecverify: argument validation, launch
// planning, workspace layout and dispatch of the gfx950 kernels.  Every
// check runs before anything is enqueued; a rejected call writes nothing.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "specverify.h"

#include <cstddef>
#include "sv_kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int status, const char *fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return status;
}

int hip_fail(hipError_t e, const char *what)
{
    return fail(SV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------- device check

constexpr int kMaxDevices = 64;
std::once_flag g_arch_once[kMaxDevices];
int g_arch_ok[kMaxDevices];

int check_device()
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SV_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::call_once(g_arch_once[dev], [dev] {
        hipDeviceProp_t prop;
        g_arch_ok[dev] = hipGetDeviceProperties(&prop, dev) == hipSuccess &&
                                 std::strncmp(prop.gcnArchName, "gfx950", 6) == 0
                             ? 1
                             : -1;
    });
    if (g_arch_ok[dev] != 1)
        return fail(SV_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
    return SV_OK;
}

// ---------------------------------------------------------------- planning

// Launch tuning, process-wide.  Every call reads it once into a Tuning and
// plans its launch and its workspace need from that copy alone, so a
// concurrent change can never make one call disagree with itself: a
// workspace sized before a change that needs more is rejected
// (SV_ERR_WORKSPACE), never overrun.
constexpr int64_t kDefaultTargetWgs = 2048;
constexpr int64_t kDefaultMinSegBytes = 32 * 1024;
std::atomic<int64_t> g_target_wgs{kDefaultTargetWgs};
std::atomic<int64_t> g_min_seg_bytes{kDefaultMinSegBytes};
constexpr int64_t kCUs = 256;

struct Tuning {
    int64_t target_wgs;
    int64_t min_seg_bytes;
};

Tuning tuning_now()
{
    return Tuning{g_target_wgs.load(std::memory_order_relaxed), g_min_seg_bytes.load(std::memory_order_relaxed)};
}

struct RowPlan {
    int segs;
    int seg_len;
};

// Launch shape of a row-streaming kernel: every row is cut into `segs`
// segments.  Rows alone fill the grid once there are target_wgs of them
// (8 workgroups per CU on 256 CUs); below that, the segment count is chosen
// among those giving at least target_wgs workgroups (and segments of at
// least min_seg_bytes) so that the workgroups fill whole rounds of the 256
// compute units as closely as possible.
RowPlan plan_rows(int64_t rows, int V, int esize, const Tuning &tu)
{
    const int64_t by_size = std::max<int64_t>(1, static_cast<int64_t>(V) * esize / tu.min_seg_bytes);
    const int64_t lo = std::min(by_size, (tu.target_wgs + rows - 1) / rows);
    const int64_t hi = std::min(by_size, 2 * lo);
    int64_t segs = lo;
    double best = -1.0;
    for (int64_t s = lo; s <= hi; ++s) {
        const int64_t w = rows * s;
        const double fill = static_cast<double>(w) / static_cast<double>((w + kCUs - 1) / kCUs * kCUs);
        if (fill > best + 1e-9) {
            best = fill;
            segs = s;
        }
    }
    // segment length: a multiple of 64 elements so that segment starts keep
    // the 16-byte alignment of the row
    int64_t seg_len = (V + segs - 1) / segs;
    seg_len = (seg_len + 63) / 64 * 64;
    segs = (V + seg_len - 1) / seg_len;
    return RowPlan{static_cast<int>(segs), static_cast<int>(seg_len)};
}

// Launch shape of the one-wave-per-item rejection statistics kernel: each
// row is cut into `segs` pieces so that the items about fill the wave slots
// of the chip (4 * target_wgs waves: 32 per CU) in a single round, with
// pieces of at least min_seg_bytes / 4 and at most kMaxSegs per row.
RowPlan plan_items(int64_t rows, int V, int esize, const Tuning &tu)
{
    const int64_t slots = 4 * tu.target_wgs;
    const int64_t by_size = std::max<int64_t>(1, static_cast<int64_t>(V) * esize * 4 / tu.min_seg_bytes);
    int64_t segs = std::max<int64_t>(1, slots / rows);
    segs = std::min<int64_t>(segs, std::min<int64_t>(by_size, sv::kMaxSegs));
    int64_t seg_len = (V + segs - 1) / segs;
    seg_len = (seg_len + 63) / 64 * 64;
    segs = (V + seg_len - 1) / seg_len;
    return RowPlan{static_cast<int>(segs), static_cast<int>(seg_len)};
}

size_t align_up(size_t x) { return (x + 255) / 256 * 256; }

// Byte offsets of the workspace pieces of one call.
struct ArgLayout {
    size_t partial, total;
};

ArgLayout arg_layout(int64_t B, int64_t rows_per_seq, const RowPlan &pl)
{
    ArgLayout L{};
    L.partial = 0;
    L.total = align_up(sizeof(sv::ArgPartial) * B * rows_per_seq * pl.segs);
    return L;
}

// The rejection workspace: the sub-chunk masses first (their place and size
// depend on B and V only, so the shard calls that write and read them agree
// whatever the launch plan), then the statistics partials and the sequence
// states.
struct RejLayout {
    size_t cmass, partial, seq, total;
};

int64_t sample_blocks(int V) { return (static_cast<int64_t>(V) + sv::kRejSub - 1) / sv::kRejSub; }

RejLayout rej_layout(int64_t B, int64_t K, int V, const RowPlan &pl)
{
    const int64_t rows = B * (2 * K + 1);
    RejLayout L{};
    size_t off = 0;
    L.cmass = off;
    off = align_up(off + sizeof(sv::ChunkMass) * B * sample_blocks(V));
    L.partial = off;
    off = align_up(off + sizeof(sv::SoftPartial) * rows * pl.segs);
    L.seq = off;
    off = align_up(off + sizeof(sv::SeqState) * B);
    L.total = off;
    return L;
}

int esize_of(int dtype) { return dtype == SV_BF16 ? 2 : 4; }

bool misaligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) != 0; }

template <typename T>
T *at(void *base, size_t off)
{
    return reinterpret_cast<T *>(static_cast<char *>(base) + off);
}

int check_logits(const void *logits, int dtype, int64_t row_stride, int V, const char *name)
{
    if (dtype != SV_F32 && dtype != SV_BF16)
        return fail(SV_ERR_INVALID_ARG, "dtype %d is neither SV_F32 nor SV_BF16", dtype);
    if (!logits)
        return fail(SV_ERR_INVALID_ARG, "%s is NULL", name);
    if (misaligned(logits, esize_of(dtype)))
        return fail(SV_ERR_INVALID_ARG, "%s is not aligned to its element size", name);
    if (row_stride < V)
        return fail(SV_ERR_INVALID_ARG, "row_stride %lld < V %d", (long long)row_stride, V);
    return SV_OK;
}

int check_workspace(void *ws, size_t have, size_t need)
{
    if (!ws)
        return fail(SV_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (misaligned(ws, 16))
        return fail(SV_ERR_WORKSPACE, "workspace is not 16-byte aligned");
    if (have < need)
        return fail(SV_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
    return SV_OK;
}

int check_sizes(int32_t B, int32_t K, int32_t V)
{
    if (B < 1)
        return fail(SV_ERR_INVALID_ARG, "B = %d < 1", B);
    if (K < 0)
        return fail(SV_ERR_INVALID_ARG, "K = %d < 0", K);
    if (V < 1)
        return fail(SV_ERR_INVALID_ARG, "V = %d < 1", V);
    if (K > SV_MAX_DRAFTS)
        return fail(SV_ERR_UNSUPPORTED, "K = %d above %d", K, SV_MAX_DRAFTS);
    if (V > SV_MAX_V)
        return fail(SV_ERR_UNSUPPORTED, "V = %d above %d", V, SV_MAX_V);
    return SV_OK;
}

int check_grid(int64_t wgs)
{
    if (wgs > 0x7fffffffLL)
        return fail(SV_ERR_UNSUPPORTED, "launch of %lld workgroups is too large", (long long)wgs);
    return SV_OK;
}

} // namespace

// ======================================================================= ABI

extern "C" {

int sv_abi_version(void) { return SV_ABI_VERSION; }

const char *sv_status_string(int status)
{
    switch (status) {
    case SV_OK: return "SV_OK";
    case SV_ERR_INVALID_ARG: return "SV_ERR_INVALID_ARG";
    case SV_ERR_UNSUPPORTED: return "SV_ERR_UNSUPPORTED";
    case SV_ERR_WORKSPACE: return "SV_ERR_WORKSPACE";
    case SV_ERR_HIP: return "SV_ERR_HIP";
    default: return "SV_ERR_UNKNOWN";
    }
}

const char *sv_last_error_message(void) { return g_err.c_str(); }

int sv_set_tuning(int32_t key, int64_t value)
{
    if (key == SV_TUNE_TARGET_WORKGROUPS) {
        g_target_wgs.store(value > 0 ? value : kDefaultTargetWgs, std::memory_order_relaxed);
        return SV_OK;
    }
    if (key == SV_TUNE_MIN_SEGMENT_BYTES) {
        g_min_seg_bytes.store(value > 0 ? value : kDefaultMinSegBytes, std::memory_order_relaxed);
        return SV_OK;
    }
    return fail(SV_ERR_INVALID_ARG, "unknown tuning key %d", key);
}

// ------------------------------------------------------------------ greedy

size_t sv_greedy_workspace_bytes(int32_t B, int32_t K, int32_t V)
{
    if (B < 1 || K < 0 || V < 1)
        return 0;
    const Tuning tu = tuning_now();
    const RowPlan a = plan_rows(static_cast<int64_t>(B) * (K + 1), V, 2, tu);
    const RowPlan b = plan_rows(static_cast<int64_t>(B) * (K + 1), V, 4, tu);
    const size_t x = arg_layout(B, K + 1, a).total, y = arg_layout(B, K + 1, b).total;
    return x > y ? x : y;
}

int sv_verify_greedy(const void *logits, int32_t dtype, int64_t row_stride,
                     const int32_t *draft, const int32_t *draft_len,
                     int32_t B, int32_t K, int32_t V,
                     int32_t *accepted, int32_t *emitted, int32_t *argmax_out,
                     uint32_t *flags, int64_t *stats,
                     void *workspace, size_t workspace_bytes, void *stream)
{
    int st;
    if ((st = check_sizes(B, K, V)) != SV_OK)
        return st;
    if ((st = check_logits(logits, dtype, row_stride, V, "logits")) != SV_OK)
        return st;
    if (K > 0 && !draft)
        return fail(SV_ERR_INVALID_ARG, "draft is NULL");
    if (!accepted || !emitted)
        return fail(SV_ERR_INVALID_ARG, "accepted and emitted are required");
    const int64_t rows = static_cast<int64_t>(B) * (K + 1);
    const RowPlan pl = plan_rows(rows, V, esize_of(dtype), tuning_now());
    const ArgLayout L = arg_layout(B, K + 1, pl);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK)
        return st;
    if ((st = check_grid(rows * pl.segs)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::ArgVerifyParams p{};
    p.logits = logits;
    p.row_stride = row_stride;
    p.B = B;
    p.V = V;
    p.rows_per_seq = K + 1;
    p.segs = pl.segs;
    p.seg_len = pl.seg_len;
    p.draft = draft;
    p.draft_len = draft_len;
    p.K = K;
    p.stats = stats;
    p.accepted = accepted;
    p.emitted = emitted;
    p.argmax_out = argmax_out;
    p.flags = flags;
    p.partial = at<sv::ArgPartial>(workspace, L.partial);
    hipError_t e = sv::launch_greedy(p, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "greedy launch");
    return SV_OK;
}

// ------------------------------------------------------------------ tree

size_t sv_tree_workspace_bytes(int32_t B, int32_t N, int32_t V)
{
    if (B < 1 || N < 1 || V < 1)
        return 0;
    const Tuning tu = tuning_now();
    const RowPlan a = plan_rows(static_cast<int64_t>(B) * N, V, 2, tu);
    const RowPlan b = plan_rows(static_cast<int64_t>(B) * N, V, 4, tu);
    const size_t x = arg_layout(B, N, a).total, y = arg_layout(B, N, b).total;
    return x > y ? x : y;
}

int sv_verify_tree(const void *logits, int32_t dtype, int64_t row_stride,
                   const int32_t *parent, const int32_t *token,
                   int32_t B, int32_t N, int32_t V,
                   int32_t *accepted, int32_t *path, int32_t *emitted,
                   int32_t *argmax_out, uint32_t *flags,
                   void *workspace, size_t workspace_bytes, void *stream)
{
    int st;
    if (B < 1)
        return fail(SV_ERR_INVALID_ARG, "B = %d < 1", B);
    if (N < 1)
        return fail(SV_ERR_INVALID_ARG, "N = %d < 1", N);
    if (V < 1)
        return fail(SV_ERR_INVALID_ARG, "V = %d < 1", V);
    if (N > SV_MAX_TREE_NODES)
        return fail(SV_ERR_UNSUPPORTED, "N = %d above %d", N, SV_MAX_TREE_NODES);
    if (V > SV_MAX_V)
        return fail(SV_ERR_UNSUPPORTED, "V = %d above %d", V, SV_MAX_V);
    if ((st = check_logits(logits, dtype, row_stride, V, "logits")) != SV_OK)
        return st;
    if (!parent || !token)
        return fail(SV_ERR_INVALID_ARG, "parent and token are required");
    if (!accepted || !path || !emitted)
        return fail(SV_ERR_INVALID_ARG, "accepted, path and emitted are required");
    const int64_t rows = static_cast<int64_t>(B) * N;
    const RowPlan pl = plan_rows(rows, V, esize_of(dtype), tuning_now());
    const ArgLayout L = arg_layout(B, N, pl);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK)
        return st;
    if ((st = check_grid(rows * pl.segs)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::ArgVerifyParams p{};
    p.logits = logits;
    p.row_stride = row_stride;
    p.B = B;
    p.V = V;
    p.rows_per_seq = N;
    p.segs = pl.segs;
    p.seg_len = pl.seg_len;
    p.parent = parent;
    p.token = token;
    p.path = path;
    p.accepted = accepted;
    p.emitted = emitted;
    p.argmax_out = argmax_out;
    p.flags = flags;
    p.partial = at<sv::ArgPartial>(workspace, L.partial);
    hipError_t e = sv::launch_tree(p, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "tree launch");
    return SV_OK;
}

// ------------------------------------------------------------------ vocabulary shards

static_assert(sizeof(sv_argmax_partial) == sizeof(sv::ArgPartial) &&
                  offsetof(sv_argmax_partial, value) == offsetof(sv::ArgPartial, v) &&
                  offsetof(sv_argmax_partial, index) == offsetof(sv::ArgPartial, i),
              "the public shard partial is the kernels' partial");
static_assert(SV_NO_INDEX == 0x7fffffff, "the kernels' 'no index' value");

size_t sv_argmax_shard_workspace_bytes(int32_t rows, int32_t V)
{
    if (rows < 1 || V < 1)
        return 0;
    const Tuning tu = tuning_now();
    const RowPlan a = plan_rows(rows, V, 2, tu);
    const RowPlan b = plan_rows(rows, V, 4, tu);
    const size_t x = arg_layout(1, rows, a).total, y = arg_layout(1, rows, b).total;
    return x > y ? x : y;
}

int sv_argmax_shard(const void *logits, int32_t dtype, int64_t row_stride,
                    int32_t rows, int32_t V, int32_t v_offset,
                    sv_argmax_partial *out,
                    void *workspace, size_t workspace_bytes, void *stream)
{
    int st;
    if (rows < 1)
        return fail(SV_ERR_INVALID_ARG, "rows = %d < 1", rows);
    if (V < 1)
        return fail(SV_ERR_INVALID_ARG, "V = %d < 1", V);
    if (v_offset < 0)
        return fail(SV_ERR_INVALID_ARG, "v_offset = %d < 0", v_offset);
    if (static_cast<int64_t>(v_offset) + V > SV_MAX_V)
        return fail(SV_ERR_UNSUPPORTED, "v_offset + V = %lld above %d",
                    static_cast<long long>(v_offset) + V, SV_MAX_V);
    if ((st = check_logits(logits, dtype, row_stride, V, "logits")) != SV_OK)
        return st;
    if (!out || misaligned(out, 8))
        return fail(SV_ERR_INVALID_ARG, "out must be non-NULL and 8-byte aligned");
    const RowPlan pl = plan_rows(rows, V, esize_of(dtype), tuning_now());
    const ArgLayout L = arg_layout(1, rows, pl);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK)
        return st;
    if ((st = check_grid(static_cast<int64_t>(rows) * pl.segs)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::ArgVerifyParams p{};
    p.logits = logits;
    p.row_stride = row_stride;
    p.B = 1;
    p.V = V;
    p.rows_per_seq = rows;
    p.segs = pl.segs;
    p.seg_len = pl.seg_len;
    p.partial = at<sv::ArgPartial>(workspace, L.partial);
    p.v_offset = v_offset;
    p.shard_out = reinterpret_cast<sv::ArgPartial *>(out);
    hipError_t e = sv::launch_argmax_shard(p, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "shard argmax launch");
    return SV_OK;
}

namespace {

int check_partials(const sv_argmax_partial *partials, int32_t P)
{
    if (P < 1)
        return fail(SV_ERR_INVALID_ARG, "P = %d < 1", P);
    if (P > SV_MAX_SHARDS)
        return fail(SV_ERR_UNSUPPORTED, "P = %d above %d", P, SV_MAX_SHARDS);
    if (!partials || misaligned(partials, 8))
        return fail(SV_ERR_INVALID_ARG, "partials must be non-NULL and 8-byte aligned");
    return SV_OK;
}

} // namespace

int sv_verify_greedy_partials(const sv_argmax_partial *partials, int32_t P,
                              const int32_t *draft, const int32_t *draft_len,
                              int32_t B, int32_t K, int32_t V,
                              int32_t *accepted, int32_t *emitted, int32_t *argmax_out,
                              uint32_t *flags, int64_t *stats, void *stream)
{
    int st;
    if ((st = check_sizes(B, K, V)) != SV_OK)
        return st;
    if ((st = check_partials(partials, P)) != SV_OK)
        return st;
    if (K > 0 && !draft)
        return fail(SV_ERR_INVALID_ARG, "draft is NULL");
    if (!accepted || !emitted)
        return fail(SV_ERR_INVALID_ARG, "accepted and emitted are required");
    if ((st = check_device()) != SV_OK)
        return st;

    sv::ArgVerifyParams p{};
    p.B = B;
    p.V = V;
    p.rows_per_seq = K + 1;
    p.segs = P;
    p.partial_in = reinterpret_cast<const sv::ArgPartial *>(partials);
    p.part_row_step = 1;
    p.part_seg_step = static_cast<int64_t>(B) * (K + 1);
    p.draft = draft;
    p.draft_len = draft_len;
    p.K = K;
    p.stats = stats;
    p.accepted = accepted;
    p.emitted = emitted;
    p.argmax_out = argmax_out;
    p.flags = flags;
    hipError_t e = sv::launch_greedy_scan(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "greedy scan launch");
    return SV_OK;
}

int sv_verify_tree_partials(const sv_argmax_partial *partials, int32_t P,
                            const int32_t *parent, const int32_t *token,
                            int32_t B, int32_t N, int32_t V,
                            int32_t *accepted, int32_t *path, int32_t *emitted,
                            int32_t *argmax_out, uint32_t *flags, void *stream)
{
    int st;
    if (B < 1)
        return fail(SV_ERR_INVALID_ARG, "B = %d < 1", B);
    if (N < 1)
        return fail(SV_ERR_INVALID_ARG, "N = %d < 1", N);
    if (V < 1)
        return fail(SV_ERR_INVALID_ARG, "V = %d < 1", V);
    if (N > SV_MAX_TREE_NODES)
        return fail(SV_ERR_UNSUPPORTED, "N = %d above %d", N, SV_MAX_TREE_NODES);
    if (V > SV_MAX_V)
        return fail(SV_ERR_UNSUPPORTED, "V = %d above %d", V, SV_MAX_V);
    if ((st = check_partials(partials, P)) != SV_OK)
        return st;
    if (!parent || !token)
        return fail(SV_ERR_INVALID_ARG, "parent and token are required");
    if (!accepted || !path || !emitted)
        return fail(SV_ERR_INVALID_ARG, "accepted, path and emitted are required");
    if ((st = check_device()) != SV_OK)
        return st;

    sv::ArgVerifyParams p{};
    p.B = B;
    p.V = V;
    p.rows_per_seq = N;
    p.segs = P;
    p.partial_in = reinterpret_cast<const sv::ArgPartial *>(partials);
    p.part_row_step = 1;
    p.part_seg_step = static_cast<int64_t>(B) * N;
    p.parent = parent;
    p.token = token;
    p.path = path;
    p.accepted = accepted;
    p.emitted = emitted;
    p.argmax_out = argmax_out;
    p.flags = flags;
    hipError_t e = sv::launch_tree_scan(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "tree scan launch");
    return SV_OK;
}

// ------------------------------------------------------------------ device array
//
// The workspace of sv_verify_rejection_noalloc: one array per GPU, loaded
// with the library's code on that GPU and kept until the process ends, for
// callers that cannot allocate.  In host code `scratch` only names the
// symbol; its address on a device comes from hipGetSymbolAddress, taken once
// per device with that device current (the calling thread's device at the
// entry point's first call on it), and only that address is passed on.

static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr size_t kScratchBytes = SV_NOALLOC_WORKSPACE_BYTES;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The array's address on the current device (after check_device).
int scratch_for_device(void **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(SV_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = p;
    });
    if (g_scratch_err[dev] != hipSuccess)
        return hip_fail(g_scratch_err[dev], "hipGetSymbolAddress of the device array");
    if (!g_scratch_ptr[dev])
        return fail(SV_ERR_HIP, "the device array has no address on device %d", dev);
    *out = g_scratch_ptr[dev];
    return SV_OK;
}

} // namespace

// ------------------------------------------------------------------ rejection

namespace {

// Temperature constants of a rejection-sampling launch: 1/T in fp32 and
// fp64, and log2(e)/T split into a 16-bit head and a remainder times ln 2
// (the bf16 statistics kernel's exact-product exp).
void set_temperature(sv::RejectParams &p, float temperature)
{
    p.inv_t_d = 1.0 / static_cast<double>(temperature);
    p.inv_t = static_cast<float>(p.inv_t_d);
    const double c = 1.4426950408889634 / static_cast<double>(temperature);   // log2(e) / T
    int ex = 0;
    const double m = std::frexp(c, &ex);                      // c = m 2^ex, m in [0.5, 1)
    const double c1 = std::ldexp(std::nearbyint(std::ldexp(m, 16)), ex - 16);
    p.split_c1 = static_cast<float>(c1);                      // exact: 16 significant bits
    p.split_k2 = static_cast<float>((c - c1) * 0.69314718055994531);
    p.split_ok = c >= 0x1p-60 && c <= 0x1p60;
}

// Logit rows of one call (all rows, or one vocabulary shard's columns).
void set_rows(sv::RejectParams &p, const void *target_logits, const void *draft_logits, int dtype,
              int64_t row_stride, int32_t B, int32_t K, int32_t V)
{
    p.target = target_logits;
    p.draftl = K > 0 ? draft_logits : target_logits;
    p.row_stride = row_stride;
    p.B = B;
    p.K = K;
    p.V = V;
    p.v_full = V;
    p.nchunks = (V + sv::kRejChunk - 1) / sv::kRejChunk;
    p.nsub = static_cast<int32_t>(sample_blocks(V));
    const int64_t esize = esize_of(dtype);
    p.vec_ok = !misaligned(target_logits, 16) && (K == 0 || !misaligned(draft_logits, 16)) &&
               (row_stride * esize) % 16 == 0 && V % (16 / esize) == 0;
}

int check_temperature(float temperature)
{
    if (!(std::isfinite(temperature) && temperature > 0.0f))
        return fail(SV_ERR_INVALID_ARG, "temperature must be finite and > 0");
    return SV_OK;
}

} // namespace

size_t sv_rejection_workspace_bytes(int32_t B, int32_t K, int32_t V)
{
    if (B < 1 || K < 0 || V < 1)
        return 0;
    const int64_t rows = static_cast<int64_t>(B) * (2 * K + 1);
    const Tuning tu = tuning_now();
    const RowPlan a = plan_items(rows, V, 2, tu);
    const RowPlan b = plan_items(rows, V, 4, tu);
    const size_t x = rej_layout(B, K, V, a).total, y = rej_layout(B, K, V, b).total;
    return x > y ? x : y;
}

namespace {

int rejection_call(const void *target_logits, const void *draft_logits,
                   int32_t dtype, int64_t row_stride,
                   const int32_t *draft, const int32_t *draft_len,
                   const float *uniforms, float temperature,
                   int32_t B, int32_t K, int32_t V,
                   int32_t *accepted, int32_t *emitted,
                   float *p_draft, float *q_draft,
                   uint32_t *flags, int64_t *stats,
                   void *workspace, size_t workspace_bytes, void *stream, bool probs,
                   bool use_scratch = false)
{
    int st;
    if ((st = check_sizes(B, K, V)) != SV_OK)
        return st;
    if ((st = check_logits(target_logits, dtype, row_stride, V, "target_logits")) != SV_OK)
        return st;
    if (K > 0 && (st = check_logits(draft_logits, dtype, row_stride, V, "draft_logits")) != SV_OK)
        return st;
    if (K > 0 && !draft)
        return fail(SV_ERR_INVALID_ARG, "draft is NULL");
    if (!uniforms)
        return fail(SV_ERR_INVALID_ARG, "uniforms is NULL");
    if ((st = check_temperature(temperature)) != SV_OK)
        return st;
    if (!accepted || !emitted)
        return fail(SV_ERR_INVALID_ARG, "accepted and emitted are required");
    const int64_t rows = static_cast<int64_t>(B) * (2 * K + 1);
    const RowPlan pl = plan_items(rows, V, esize_of(dtype), tuning_now());
    const RejLayout L = rej_layout(B, K, V, pl);
    if (use_scratch && L.total > kScratchBytes)
        return fail(SV_ERR_UNSUPPORTED, "this call needs %zu bytes of workspace, above the %zu bytes of the "
                    "library's device array", L.total, kScratchBytes);
    const int nchunks = (V + sv::kRejChunk - 1) / sv::kRejChunk;
    if ((st = check_grid((rows * pl.segs + 3) / 4)) != SV_OK)
        return st;
    if ((st = check_grid(static_cast<int64_t>(B) * nchunks)) != SV_OK)
        return st;
    if (use_scratch) {
        if ((st = check_device()) != SV_OK)
            return st;
        if ((st = scratch_for_device(&workspace)) != SV_OK)
            return st;
        workspace_bytes = kScratchBytes;
    }
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::RejectParams p{};
    set_rows(p, target_logits, draft_logits, dtype, row_stride, B, K, V);
    p.segs = pl.segs;
    p.seg_len = pl.seg_len;
    p.part_row_step = pl.segs;
    p.part_seg_step = 1;
    p.capture_x = 1;
    set_temperature(p, temperature);
    p.draft = K > 0 ? draft : accepted;
    p.draft_len = draft_len ? draft_len : accepted;
    p.has_len = draft_len != nullptr;
    p.u = uniforms;
    p.accepted = accepted;
    p.emitted = emitted;
    p.p_draft = p_draft;
    p.q_draft = q_draft;
    p.flags = flags;
    p.stats = stats;
    p.partial = at<sv::SoftPartial>(workspace, L.partial);
    p.seq = at<sv::SeqState>(workspace, L.seq);
    p.cmass = at<sv::ChunkMass>(workspace, L.cmass);
    p.probs = probs;
    hipError_t e = sv::launch_rejection(p, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "rejection launch");
    return SV_OK;
}

} // namespace

int sv_verify_rejection(const void *target_logits, const void *draft_logits,
                        int32_t dtype, int64_t row_stride,
                        const int32_t *draft, const int32_t *draft_len,
                        const float *uniforms, float temperature,
                        int32_t B, int32_t K, int32_t V,
                        int32_t *accepted, int32_t *emitted,
                        float *p_draft, float *q_draft,
                        uint32_t *flags, int64_t *stats,
                        void *workspace, size_t workspace_bytes, void *stream)
{
    return rejection_call(target_logits, draft_logits, dtype, row_stride, draft, draft_len, uniforms,
                          temperature, B, K, V, accepted, emitted, p_draft, q_draft, flags, stats,
                          workspace, workspace_bytes, stream, false);
}

int sv_verify_rejection_probs(const float *target_probs, const float *draft_probs,
                              int64_t row_stride,
                              const int32_t *draft, const int32_t *draft_len,
                              const float *uniforms,
                              int32_t B, int32_t K, int32_t V,
                              int32_t *accepted, int32_t *emitted,
                              float *p_draft, float *q_draft,
                              uint32_t *flags, int64_t *stats,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    return rejection_call(target_probs, draft_probs, SV_F32, row_stride, draft, draft_len, uniforms,
                          1.0f, B, K, V, accepted, emitted, p_draft, q_draft, flags, stats,
                          workspace, workspace_bytes, stream, true);
}

int sv_verify_rejection_noalloc(const void *target_logits, const void *draft_logits,
                                int32_t dtype, int64_t row_stride,
                                const int32_t *draft, const int32_t *draft_len,
                                const float *uniforms, float temperature,
                                int32_t B, int32_t K, int32_t V,
                                int32_t *accepted, int32_t *emitted,
                                float *p_draft, float *q_draft,
                                uint32_t *flags, int64_t *stats, void *stream)
{
    return rejection_call(target_logits, draft_logits, dtype, row_stride, draft, draft_len, uniforms,
                          temperature, B, K, V, accepted, emitted, p_draft, q_draft, flags, stats,
                          nullptr, 0, stream, false, true);
}

// ------------------------------------------------------- rejection, sharded

static_assert(sizeof(sv_softmax_partial) == sizeof(sv::SoftPartial), "partial layout");
static_assert(sizeof(sv_rejection_state) == sizeof(sv::SeqState), "state layout");
static_assert(sizeof(sv_sample_mass) == sizeof(sv::ChunkMass), "mass layout");
static_assert(SV_SAMPLE_BLOCK == sv::kRejSub, "the documented mass records are the sub-chunk masses");
static_assert(SV_MAX_REJECT_SHARDS <= sv::kMaxSegs, "shards merge like row segments");

namespace {

int check_shard_rows(const void *target_logits, const void *draft_logits, int32_t dtype,
                     int64_t row_stride, int32_t B, int32_t K, int32_t V, int32_t v_offset)
{
    int st;
    if ((st = check_sizes(B, K, V)) != SV_OK)
        return st;
    if (v_offset < 0)
        return fail(SV_ERR_INVALID_ARG, "v_offset = %d < 0", v_offset);
    if (static_cast<int64_t>(v_offset) + V > SV_MAX_V)
        return fail(SV_ERR_UNSUPPORTED, "v_offset + V = %lld above %d",
                    static_cast<long long>(v_offset) + V, SV_MAX_V);
    if ((st = check_logits(target_logits, dtype, row_stride, V, "target_logits")) != SV_OK)
        return st;
    if (K > 0 && (st = check_logits(draft_logits, dtype, row_stride, V, "draft_logits")) != SV_OK)
        return st;
    return SV_OK;
}

int check_shard_count(int32_t P)
{
    if (P < 1)
        return fail(SV_ERR_INVALID_ARG, "P = %d < 1", P);
    if (P > SV_MAX_REJECT_SHARDS)
        return fail(SV_ERR_UNSUPPORTED, "P = %d above %d", P, SV_MAX_REJECT_SHARDS);
    return SV_OK;
}

} // namespace

size_t sv_rejection_shard_workspace_bytes(int32_t B, int32_t K, int32_t V)
{
    return sv_rejection_workspace_bytes(B, K, V);
}

int sv_rejection_shard_stats(const void *target_logits, const void *draft_logits,
                             int32_t dtype, int64_t row_stride,
                             const int32_t *draft, const int32_t *draft_len, float temperature,
                             int32_t B, int32_t K, int32_t V, int32_t v_offset,
                             sv_softmax_partial *out,
                             void *workspace, size_t workspace_bytes, void *stream)
{
    int st;
    if ((st = check_shard_rows(target_logits, draft_logits, dtype, row_stride, B, K, V, v_offset)) != SV_OK)
        return st;
    if (K > 0 && !draft)
        return fail(SV_ERR_INVALID_ARG, "draft is NULL");
    if ((st = check_temperature(temperature)) != SV_OK)
        return st;
    if (!out || misaligned(out, 8))
        return fail(SV_ERR_INVALID_ARG, "out must be non-NULL and 8-byte aligned");
    const int64_t rows = static_cast<int64_t>(B) * (2 * K + 1);
    const RowPlan pl = plan_items(rows, V, esize_of(dtype), tuning_now());
    const RejLayout L = rej_layout(B, K, V, pl);
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK)
        return st;
    if ((st = check_grid((rows * pl.segs + 3) / 4)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::RejectParams p{};
    set_rows(p, target_logits, draft_logits, dtype, row_stride, B, K, V);
    p.segs = pl.segs;
    p.seg_len = pl.seg_len;
    set_temperature(p, temperature);
    p.v_offset = v_offset;
    p.capture_x = 1;
    p.draft = K > 0 ? draft : reinterpret_cast<const int32_t *>(out);
    p.draft_len = draft_len ? draft_len : reinterpret_cast<const int32_t *>(out);
    p.has_len = draft_len != nullptr;
    p.partial = at<sv::SoftPartial>(workspace, L.partial);
    hipError_t e = sv::launch_rejection_shard_stats(p, dtype, reinterpret_cast<sv::SoftPartial *>(out),
                                                    static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "shard statistics launch");
    return SV_OK;
}

int sv_verify_rejection_partials(const sv_softmax_partial *partials, int32_t P,
                                 const int32_t *draft, const int32_t *draft_len,
                                 const float *uniforms, float temperature,
                                 int32_t B, int32_t K, int32_t V,
                                 int32_t *accepted, float *p_draft, float *q_draft,
                                 uint32_t *flags, int64_t *stats,
                                 sv_rejection_state *state, void *stream)
{
    int st;
    if ((st = check_shard_count(P)) != SV_OK)
        return st;
    if (!partials || misaligned(partials, 8))
        return fail(SV_ERR_INVALID_ARG, "partials must be non-NULL and 8-byte aligned");
    if ((st = check_sizes(B, K, V)) != SV_OK)
        return st;
    if (K > 0 && !draft)
        return fail(SV_ERR_INVALID_ARG, "draft is NULL");
    if (!uniforms)
        return fail(SV_ERR_INVALID_ARG, "uniforms is NULL");
    if ((st = check_temperature(temperature)) != SV_OK)
        return st;
    if (!accepted || !state || misaligned(state, 8))
        return fail(SV_ERR_INVALID_ARG, "accepted and an 8-byte aligned state are required");
    if ((st = check_device()) != SV_OK)
        return st;

    sv::RejectParams p{};
    p.B = B;
    p.K = K;
    p.V = V;
    p.v_full = V;
    p.segs = P;
    p.part_row_step = 1;
    p.part_seg_step = static_cast<int64_t>(B) * (2 * K + 1);
    set_temperature(p, temperature);
    p.draft = K > 0 ? draft : accepted;
    p.draft_len = draft_len ? draft_len : accepted;
    p.has_len = draft_len != nullptr;
    p.u = uniforms;
    p.accepted = accepted;
    p.p_draft = p_draft;
    p.q_draft = q_draft;
    p.flags = flags;
    p.stats = stats;
    p.partial = const_cast<sv::SoftPartial *>(reinterpret_cast<const sv::SoftPartial *>(partials));
    p.seq = reinterpret_cast<sv::SeqState *>(state);
    hipError_t e = sv::launch_rejection_decide(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "accept scan launch");
    return SV_OK;
}

int sv_rejection_shard_mass(const void *target_logits, const void *draft_logits,
                            int32_t dtype, int64_t row_stride,
                            const sv_rejection_state *state, float temperature,
                            int32_t B, int32_t K, int32_t V,
                            sv_sample_mass *out,
                            void *workspace, size_t workspace_bytes, void *stream)
{
    int st;
    if ((st = check_shard_rows(target_logits, draft_logits, dtype, row_stride, B, K, V, 0)) != SV_OK)
        return st;
    if ((st = check_temperature(temperature)) != SV_OK)
        return st;
    if (!state || misaligned(state, 8))
        return fail(SV_ERR_INVALID_ARG, "state must be non-NULL and 8-byte aligned");
    if (!out || misaligned(out, 8))
        return fail(SV_ERR_INVALID_ARG, "out must be non-NULL and 8-byte aligned");
    const int64_t rows = static_cast<int64_t>(B) * (2 * K + 1);
    const RejLayout L = rej_layout(B, K, V, plan_items(rows, V, esize_of(dtype), tuning_now()));
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK)
        return st;
    const int nchunks = (V + sv::kRejChunk - 1) / sv::kRejChunk;
    if ((st = check_grid(static_cast<int64_t>(B) * nchunks)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::RejectParams p{};
    set_rows(p, target_logits, draft_logits, dtype, row_stride, B, K, V);
    set_temperature(p, temperature);
    p.seq = const_cast<sv::SeqState *>(reinterpret_cast<const sv::SeqState *>(state));
    p.cmass = at<sv::ChunkMass>(workspace, L.cmass);
    p.mass_out = reinterpret_cast<sv::ChunkMass *>(out);
    hipError_t e = sv::launch_rejection_shard_mass(p, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "shard mass launch");
    return SV_OK;
}

int sv_rejection_shard_sample(const void *target_logits, const void *draft_logits,
                              int32_t dtype, int64_t row_stride,
                              const int32_t *draft, const float *uniforms,
                              const sv_rejection_state *state,
                              const sv_sample_mass *masses, int32_t P, int32_t shard,
                              float temperature, int32_t B, int32_t K, int32_t V, int32_t v_offset,
                              int32_t *emitted,
                              void *workspace, size_t workspace_bytes, void *stream)
{
    int st;
    if ((st = check_shard_rows(target_logits, draft_logits, dtype, row_stride, B, K, V, v_offset)) != SV_OK)
        return st;
    if ((st = check_shard_count(P)) != SV_OK)
        return st;
    if (shard < 0 || shard >= P)
        return fail(SV_ERR_INVALID_ARG, "shard = %d outside [0, %d)", shard, P);
    if (K > 0 && !draft)
        return fail(SV_ERR_INVALID_ARG, "draft is NULL");
    if (!uniforms)
        return fail(SV_ERR_INVALID_ARG, "uniforms is NULL");
    if ((st = check_temperature(temperature)) != SV_OK)
        return st;
    if (!state || misaligned(state, 8) || !masses || misaligned(masses, 8))
        return fail(SV_ERR_INVALID_ARG, "state and masses must be non-NULL and 8-byte aligned");
    if (!emitted)
        return fail(SV_ERR_INVALID_ARG, "emitted is NULL");
    const int64_t rows = static_cast<int64_t>(B) * (2 * K + 1);
    const RejLayout L = rej_layout(B, K, V, plan_items(rows, V, esize_of(dtype), tuning_now()));
    if ((st = check_workspace(workspace, workspace_bytes, L.total)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::RejectParams p{};
    set_rows(p, target_logits, draft_logits, dtype, row_stride, B, K, V);
    set_temperature(p, temperature);
    p.v_offset = v_offset;
    p.draft = K > 0 ? draft : emitted;
    p.u = uniforms;
    p.emitted = emitted;
    p.seq = const_cast<sv::SeqState *>(reinterpret_cast<const sv::SeqState *>(state));
    p.cmass = at<sv::ChunkMass>(workspace, L.cmass);
    p.shard_mass = reinterpret_cast<const sv::ChunkMass *>(masses);
    p.shard_count = P;
    p.shard_index = shard;
    hipError_t e = sv::launch_rejection_shard_sample(p, dtype, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "shard sample launch");
    return SV_OK;
}

// ------------------------------------------------------------------ probe

int sv_read_probe(const void *buf, size_t bytes, uint32_t *out, void *stream)
{
    int st;
    if (!buf || !out)
        return fail(SV_ERR_INVALID_ARG, "buf and out are required");
    if (bytes < 16 || bytes % 16 != 0 || misaligned(buf, 16))
        return fail(SV_ERR_INVALID_ARG, "bytes must be a positive multiple of 16 and buf 16-byte aligned");
    const int64_t wgs = tuning_now().target_wgs;
    if (bytes / 4 > (static_cast<size_t>(1) << 30) * static_cast<size_t>(wgs))
        return fail(SV_ERR_UNSUPPORTED, "bytes too large");
    if ((st = check_device()) != SV_OK)
        return st;
    hipError_t e = sv::launch_read_probe(buf, static_cast<int64_t>(bytes), out, static_cast<int>(wgs),
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "probe launch");
    return SV_OK;
}

// ------------------------------------------------------------------ suffix

namespace {

int suffix_chunks(int64_t n) { return static_cast<int>((n + sv::kSfxChunk - 1) / sv::kSfxChunk); }

} // namespace

size_t sv_suffix_workspace_bytes(int32_t B, int64_t ctx_stride, int64_t H)
{
    if (B < 1 || ctx_stride < 1 || ctx_stride > SV_MAX_CONTEXT || H < 0 || H > SV_MAX_CONTEXT)
        return 0;
    return align_up(sizeof(sv::SuffixScanRec) * static_cast<size_t>(B) *
                    static_cast<size_t>(suffix_chunks(ctx_stride) + suffix_chunks(H)));
}

int sv_suffix_propose(const int32_t *tokens, int64_t ctx_stride, const int32_t *lengths, int32_t B,
                      const int32_t *history, int64_t H,
                      int32_t m_min, int32_t m_max, int32_t K, double min_prob,
                      int32_t *proposal, int32_t *proposal_len, double *score,
                      int32_t *match_len, int32_t *source, uint32_t *flags,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    int st;
    if (B < 1)
        return fail(SV_ERR_INVALID_ARG, "B = %d < 1", B);
    if (m_min < 1 || m_max < m_min)
        return fail(SV_ERR_INVALID_ARG, "need 1 <= m_min <= m_max (got %d, %d)", m_min, m_max);
    if (m_max > SV_SUFFIX_MAX_MATCH)
        return fail(SV_ERR_UNSUPPORTED, "m_max = %d above %d", m_max, SV_SUFFIX_MAX_MATCH);
    if (K < 0)
        return fail(SV_ERR_INVALID_ARG, "K = %d < 0", K);
    if (K > SV_SUFFIX_MAX_K)
        return fail(SV_ERR_UNSUPPORTED, "K = %d above %d", K, SV_SUFFIX_MAX_K);
    if (!(min_prob >= 0.0 && min_prob <= 1.0))
        return fail(SV_ERR_INVALID_ARG, "min_prob must lie in [0, 1]");
    if (ctx_stride < 1 || ctx_stride > SV_MAX_CONTEXT)
        return fail(ctx_stride < 1 ? SV_ERR_INVALID_ARG : SV_ERR_UNSUPPORTED,
                    "ctx_stride = %lld outside [1, %d]", static_cast<long long>(ctx_stride),
                    SV_MAX_CONTEXT);
    if (H < 0 || H > SV_MAX_CONTEXT)
        return fail(H < 0 ? SV_ERR_INVALID_ARG : SV_ERR_UNSUPPORTED,
                    "H = %lld outside [0, %d]", static_cast<long long>(H), SV_MAX_CONTEXT);
    if (!tokens || !lengths || !proposal_len)
        return fail(SV_ERR_INVALID_ARG, "tokens, lengths and proposal_len are required");
    if (K > 0 && !proposal)
        return fail(SV_ERR_INVALID_ARG, "proposal is NULL");
    if (H > 0 && !history)
        return fail(SV_ERR_INVALID_ARG, "history is NULL with H = %lld", static_cast<long long>(H));
    if (score && misaligned(score, 8))
        return fail(SV_ERR_INVALID_ARG, "score must be 8-byte aligned");
    if ((st = check_workspace(workspace, workspace_bytes, sv_suffix_workspace_bytes(B, ctx_stride, H))) != SV_OK)
        return st;
    const int nch_ctx = suffix_chunks(ctx_stride), nch_hist = suffix_chunks(H);
    if ((st = check_grid((static_cast<int64_t>(B) * (nch_ctx + nch_hist) + 3) / 4)) != SV_OK)
        return st;
    if ((st = check_device()) != SV_OK)
        return st;

    sv::SuffixParams p{};
    p.tokens = tokens;
    p.ctx_stride = ctx_stride;
    p.lengths = lengths;
    p.B = B;
    p.history = H > 0 ? history : tokens;
    p.H = H;
    p.m_min = m_min;
    p.m_max = m_max;
    p.K = K;
    p.min_prob = min_prob;
    p.proposal = K > 0 ? proposal : proposal_len;
    p.proposal_len = proposal_len;
    p.score = score;
    p.match_len = match_len;
    p.source = source;
    p.flags = flags;
    p.rec = static_cast<sv::SuffixScanRec *>(workspace);
    p.nch_ctx = nch_ctx;
    p.nch_hist = nch_hist;
    p.vec_ok = !misaligned(tokens, 16) && ctx_stride % 4 == 0 &&
               (H == 0 || (!misaligned(history, 16) && H % 4 == 0));
    hipError_t e = sv::launch_suffix(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "suffix launch");
    return SV_OK;
}

// ------------------------------------------------------------------ n-gram

int sv_ngram_propose(const int32_t *tokens, int64_t ctx_stride,
                     const int32_t *lengths, int32_t B,
                     int32_t n_min, int32_t n_max, int32_t K,
                     int32_t *proposal, int32_t *proposal_len,
                     int32_t *match_n, int32_t *match_pos,
                     uint32_t *flags, void *stream)
{
    if (B < 1)
        return fail(SV_ERR_INVALID_ARG, "B = %d < 1", B);
    if (n_min < 1 || n_max < n_min)
        return fail(SV_ERR_INVALID_ARG, "need 1 <= n_min <= n_max (got %d, %d)", n_min, n_max);
    if (n_max > SV_MAX_NGRAM)
        return fail(SV_ERR_UNSUPPORTED, "n_max = %d above %d", n_max, SV_MAX_NGRAM);
    if (K < 0)
        return fail(SV_ERR_INVALID_ARG, "K = %d < 0", K);
    if (K > SV_MAX_PROPOSAL)
        return fail(SV_ERR_UNSUPPORTED, "K = %d above %d", K, SV_MAX_PROPOSAL);
    if (ctx_stride < 1)
        return fail(SV_ERR_INVALID_ARG, "ctx_stride = %lld < 1", (long long)ctx_stride);
    if (ctx_stride > SV_MAX_CONTEXT)
        return fail(SV_ERR_UNSUPPORTED, "ctx_stride = %lld above %d", (long long)ctx_stride,
                    SV_MAX_CONTEXT);
    if (!tokens || !lengths)
        return fail(SV_ERR_INVALID_ARG, "tokens and lengths are required");
    if (misaligned(tokens, 4))
        return fail(SV_ERR_INVALID_ARG, "tokens is not 4-byte aligned");
    if (!proposal_len || (K > 0 && !proposal))
        return fail(SV_ERR_INVALID_ARG, "proposal and proposal_len are required");
    int st;
    if ((st = check_device()) != SV_OK)
        return st;
    sv::NgramParams p{};
    p.tokens = tokens;
    p.ctx_stride = ctx_stride;
    p.lengths = lengths;
    p.B = B;
    p.n_min = n_min;
    p.n_max = n_max;
    p.K = K;
    p.proposal = proposal;
    p.proposal_len = proposal_len;
    p.match_n = match_n;
    p.match_pos = match_pos;
    p.flags = flags;
    p.vec_ok = !misaligned(tokens, 16) && (ctx_stride % 4 == 0);
    hipError_t e = sv::launch_ngram(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return hip_fail(e, "n-gram launch");
    return SV_OK;
}

} // extern "C"

// ------------------------------------------------------------------ adaptive length
//
// [Handbook] "adaptive", the mechanism described for SGLang: after each
// verification round the mean number of accepted draft tokens per sequence
// updates an exponential moving average, and the next round's speculation
// length is one of a few fixed tiers chosen from it.  Host code only.

namespace {

// The smallest tier of at least twice the average, else the largest: as
// much room above the usual accepted run as the run itself uses.  (The
// average never exceeds the length in use, so the rule must move up before
// the average reaches the next tier, and down before it reaches 0.)
int32_t tier_for(const sv_adaptive &a)
{
    for (int32_t i = 0; i < a.ntiers; ++i)
        if (static_cast<double>(a.tiers[i]) >= 2.0 * a.ema)
            return a.tiers[i];
    return a.tiers[a.ntiers - 1];
}

} // namespace

extern "C" {

int sv_adaptive_init(sv_adaptive *a, const int32_t *tiers, int32_t ntiers, double beta, double ema0)
{
    if (!a || !tiers)
        return fail(SV_ERR_INVALID_ARG, "state and tiers are required");
    if (ntiers < 1 || ntiers > SV_MAX_TIERS)
        return fail(SV_ERR_INVALID_ARG, "ntiers = %d outside [1, %d]", ntiers, SV_MAX_TIERS);
    for (int32_t i = 0; i < ntiers; ++i) {
        if (tiers[i] < 1 || tiers[i] > SV_MAX_DRAFTS || (i > 0 && tiers[i] <= tiers[i - 1]))
            return fail(SV_ERR_INVALID_ARG,
                            "tiers must increase strictly within [1, %d] (tier %d = %d)",
                            SV_MAX_DRAFTS, i, tiers[i]);
    }
    if (!(beta > 0.0 && beta <= 1.0))
        return fail(SV_ERR_INVALID_ARG, "beta must lie in (0, 1]");
    if (!(std::isfinite(ema0) && ema0 >= 0.0))
        return fail(SV_ERR_INVALID_ARG, "ema0 must be finite and >= 0");
    a->ema = ema0;
    a->beta = beta;
    a->ntiers = ntiers;
    for (int32_t i = 0; i < SV_MAX_TIERS; ++i)
        a->tiers[i] = i < ntiers ? tiers[i] : 0;
    a->k = tier_for(*a);
    return SV_OK;
}

int sv_adaptive_update(sv_adaptive *a, double accepted_mean)
{
    if (!a || a->ntiers < 1 || a->ntiers > SV_MAX_TIERS)
        return fail(SV_ERR_INVALID_ARG, "state not initialised");
    if (!(std::isfinite(accepted_mean) && accepted_mean >= 0.0))
        return fail(SV_ERR_INVALID_ARG, "accepted_mean must be finite and >= 0");
    {
#pragma clang fp contract(off)
        a->ema = (1.0 - a->beta) * a->ema + a->beta * accepted_mean;   // two roundings, as written
    }
    a->k = tier_for(*a);
    return SV_OK;
}

} // extern "C"

// C ABI of the gfx950 SGEMM library: argument checks, kernel-variant choice
// and launch on the caller's stream.  The operation and its contract are
// documented in include/sgemm.h.
//
// The host picks between separately compiled kernel instantiations instead
// of branching inside the kernel: beta == 0 selects an epilogue that never
// reads C ("The Final Kernel: Retuning Against the Pipeline", Skipping The
// Read Of C), and shapes that are whole multiples of the block tile select
// the instantiation without edge guards.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <list>
#include <mutex>
#include <thread>
#include <utility>
#include <vector>

#include "sgemm.h"
#include "sgemm_kernels.hpp"

#define SGEMM_LIB_VERSION 1

namespace sgemm_mi355x {
// Lean direct-to-LDS kernels (sgemm_lean.hip, built with MFMA results in
// VGPRs): whole tiles only, offsets within the 31-bit buffer range.  Every
// launcher returns its launch's status.
hipError_t launch_lean_128x128x64_w2x2(const Args &a, hipStream_t stream);
hipError_t launch_lean_128x128x32_w2x2(const Args &a, hipStream_t stream);
hipError_t launch_lean_256x128x32_w4x2(const Args &a, hipStream_t stream);
hipError_t launch_lean_128x256x32_w2x4(const Args &a, hipStream_t stream);
hipError_t launch_lean_64x64x32_w4x1(const Args &a, hipStream_t stream);
hipError_t launch_lean_64x64x64_w4x1(const Args &a, hipStream_t stream);
hipError_t launch_lean_64x128x32_w2x2(const Args &a, hipStream_t stream);
hipError_t launch_lean_128x64x32_w4x1(const Args &a, hipStream_t stream);
hipError_t launch_lean_dw_128x128x32_w2x2(const Args &a, hipStream_t stream);
hipError_t launch_lean_dw_64x64x64_w4x1(const Args &a, hipStream_t stream);
hipError_t launch_lean_general(const Args &a, bool tile64, bool dw, bool ta, bool tb, int batch, hipStream_t stream);
hipError_t launch_lowp_tile(const Args &a, bool f16, int tile, bool ta, bool tb, int batch, hipStream_t stream);
hipError_t launch_lean_splitk_128x128x32_w2x2(const Args &a, int splits, hipStream_t stream);
hipError_t launch_lean_splitk_dw_64x64x64_w4x1(const Args &a, int splits, hipStream_t stream);
hipError_t launch_lean_splitk_64x64x32_w4x1(const Args &a, int splits, hipStream_t stream);
hipError_t launch_lean_splitk_64x64x64_w4x1(const Args &a, int splits, hipStream_t stream);
hipError_t launch_lean_splitk_64x128x32_w2x2(const Args &a, int splits, hipStream_t stream);
hipError_t launch_lean_splitk_128x64x32_w4x1(const Args &a, int splits, hipStream_t stream);
hipError_t launch_lean_splitk_g_64x64x64_w4x1(const Args &a, int splits, bool ta, bool tb, int batch,
                                              hipStream_t stream);
}  // namespace sgemm_mi355x

using namespace sgemm_mi355x;

namespace {

thread_local char g_last_hip_error[256] = "";

int record_hip_error(hipError_t e, const char *what) {
    snprintf(g_last_hip_error, sizeof(g_last_hip_error), "%s: %s (%d)", what,
             hipGetErrorString(e), (int)e);
    return SGEMM_STATUS_HIP_ERROR;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Process-wide tuning knobs read once from the environment (tile raster
// group height, the XCD remap, a forced split-K factor, the copy of
// unaligned transposed operands), for sweeps; defaults otherwise.
struct Knobs {
    int group_m = 8;
    int xcd_remap = 1;
    int splitk = 0;         // 0: automatic split-K factor; >= 1: forced
    int pack = 0;           // unaligned transposed operands: 0 automatic, 1 always copy, -1 never
    int tail_fill = 100;    // last-wave split: largest fill of the last wave split, percent of its slots
    Knobs() {
        if (const char *s = getenv("SGEMM_TAIL_FILL")) {
            int v = atoi(s);
            if (v >= 0 && v <= 100) tail_fill = v;
        }
        if (const char *s = getenv("SGEMM_PACK")) {
            int v = atoi(s);
            if (v >= -1 && v <= 1) pack = v;
        }
        if (const char *s = getenv("SGEMM_GROUP_M")) {
            int v = atoi(s);
            if (v >= 1 && v <= 1024) group_m = v;
        }
        if (const char *s = getenv("SGEMM_XCD_REMAP")) xcd_remap = atoi(s) != 0;
        if (const char *s = getenv("SGEMM_SPLITK")) {
            int v = atoi(s);
            if (v >= 0 && v <= 64) splitk = v;
        }
    }
};

const Knobs &knobs() {
    static const Knobs k;
    return k;
}

// Argument checks shared by every entry point.  No HIP call happens here.
int check_args(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
               const float *C, int ldc) {
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_DIM;
    const int kmin = K > 1 ? K : 1, nmin = N > 1 ? N : 1;
    if (lda < kmin || ldb < nmin || ldc < nmin) return SGEMM_STATUS_INVALID_DIM;
    if (M == 0 || N == 0) return SGEMM_STATUS_OK;
    if (C == nullptr) return SGEMM_STATUS_NULL_POINTER;
    if (K > 0 && (A == nullptr || B == nullptr)) return SGEMM_STATUS_NULL_POINTER;
    return SGEMM_STATUS_OK;
}

bool vec_ok(int K, const float *A, int lda, const float *B, int ldb, float beta, const float *C,
            int ldc) {
    (void)beta;
    const bool ab = K == 0 || (aligned16(A) && aligned16(B) && lda % 4 == 0 && ldb % 4 == 0);
    return ab && aligned16(C) && ldc % 4 == 0;
}

long ceil_div(long a, long b) { return (a + b - 1) / b; }

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool VEC>
hipError_t launch_db(const Args &a0, hipStream_t stream) {
    const Args a = tiled(a0, BM, BN);
    const bool guard = (a.M % BM) || (a.N % BN) || (a.K % BK);
    const bool beta0 = a.beta == 0.0f;
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(64 * WAVES_M * WAVES_N);
#define SGEMM_LAUNCH(G, Z) launch_k(sgemm_db_kernel<BM, BN, BK, WAVES_M, WAVES_N, VEC, G, Z>, grid, block, stream, a)
    if (guard) return beta0 ? SGEMM_LAUNCH(true, true) : SGEMM_LAUNCH(true, false);
    return beta0 ? SGEMM_LAUNCH(false, true) : SGEMM_LAUNCH(false, false);
#undef SGEMM_LAUNCH
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool VEC>
hipError_t launch_pipe(const Args &a0, hipStream_t stream) {
    const Args a = tiled(a0, BM, BN);
    const bool guard = (a.M % BM) || (a.N % BN) || (a.K % 16);
    const bool beta0 = a.beta == 0.0f;
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(64 * WAVES_M * WAVES_N);
#define SGEMM_LAUNCH(G, Z) launch_k(sgemm_pipe_kernel<BM, BN, WAVES_M, WAVES_N, VEC, G, Z>, grid, block, stream, a)
    if (guard) return beta0 ? SGEMM_LAUNCH(true, true) : SGEMM_LAUNCH(true, false);
    return beta0 ? SGEMM_LAUNCH(false, true) : SGEMM_LAUNCH(false, false);
#undef SGEMM_LAUNCH
}

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, bool VEC>
hipError_t launch_sec(const Args &a0, hipStream_t stream) {
    const Args a = tiled(a0, BM, BN);
    const bool guard = (a.M % BM) || (a.N % BN) || (a.K % BK);
    const bool beta0 = a.beta == 0.0f;
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(64 * WAVES_M * WAVES_N);
#define SGEMM_LAUNCH(G, Z) launch_k(sgemm_sec_kernel<BM, BN, BK, WAVES_M, WAVES_N, VEC, G, Z>, grid, block, stream, a)
    if (guard) return beta0 ? SGEMM_LAUNCH(true, true) : SGEMM_LAUNCH(true, false);
    return beta0 ? SGEMM_LAUNCH(false, true) : SGEMM_LAUNCH(false, false);
#undef SGEMM_LAUNCH
}

// Direct-to-LDS kernel for whole tiles; shapes that are not whole tiles
// fall back to the section-pipelined kernel of the same tile (guarded loads).
template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES>
hipError_t launch_dtl(const Args &a0, hipStream_t stream) {
    const Args a = tiled(a0, BM, BN);
    const bool whole = !(a.M % BM) && !(a.N % BN) && !(a.K % BK);
    if (!whole) return launch_sec<BM, BN, BK, WAVES_M, WAVES_N, true>(a, stream);
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n)), block(64 * WAVES_M * WAVES_N);
    if (a.beta == 0.0f)
        return launch_k(sgemm_dtl_kernel<BM, BN, BK, WAVES_M, WAVES_N, STAGES, true>, grid, block, stream, a);
    return launch_k(sgemm_dtl_kernel<BM, BN, BK, WAVES_M, WAVES_N, STAGES, false>, grid, block, stream, a);
}

typedef hipError_t (*Launcher)(const Args &, hipStream_t);

// ---------------------------------------------------------------------------
// Split-K (lean kernels).  A tile grid with fewer blocks than about two per
// compute unit leaves CUs idle while each busy CU walks all of K; splitting
// K over S blocks per tile multiplies the parallelism by S at the price of
// writing and re-reading S partial tiles.  The model below counts two
// resident blocks per CU, as for the 64x64x64 and 128x128x32 tiles (four
// waves, 64 KiB of LDS); in the automatic choice the grid splits on
// 64x64x64 tiles (128x128x32 grids it picks hold at least 256 tiles and
// never gain), and a partly filled last wave splits on either.
constexpr long kNumCUs = 256;                            // MI355X
constexpr long kTailSlots = 2 * kNumCUs;                 // resident lean blocks: two per CU
constexpr long kSplitMaxTiles = 4096;                    // tiles with counters
constexpr size_t kSplitPartialBytes = 64u << 20;         // 1024 partial tiles of 128x128, 256 of 256x256
constexpr size_t kSplitWorkspaceBytes = kSplitPartialBytes + kSplitMaxTiles * sizeof(unsigned);
static_assert(kSplitWorkspaceBytes == (size_t)SGEMM_WORKSPACE_BYTES, "workspace size in sgemm.h");

// Split factor for an M x N x K problem on bm x bn x bk tiles (1 = no
// split), for grids of fewer than one full wave of resident blocks (larger
// grids are left to the last-wave split).  Cost model, in K-tile steps of
// one block on a CU of its own (2 * bm * bn * bk flops at 1/256 of the
// 157.3 TFLOP/s peak):
//   - the busiest CU: ceil(tiles * S / 256) = r blocks of ceil(kt / S)
//     steps (a CU runs its blocks at about the same aggregate rate whether
//     it holds one or two), plus kBlockFixed steps (first loads, pipeline
//     fill, epilogue) for every pair of blocks it holds: two resident
//     blocks overlap their fixed parts;
//   - a floor set by the operand traffic of the whole grid, which every S
//     moves alike: 0.15 * tiles * kt * (bm + bn) / (bm * bn) steps;
//   - splitting at all: kSplitFixed steps (the device-scope hand-off and
//     the ticket) and kSplitPerPartial per split (the last block of a tile
//     reads the S partial tiles back one after the other).  The partials'
//     own traffic (at most 64 MiB, held in the caches) fitted to nothing
//     measurable and is left out.
// The cost is the larger of the first two plus the third.  S is the factor
// of least cost, with at least two K tiles per split (the pipeline's depth),
// at most 16, within the workspace, taken when it costs at most 95% of no
// split.  The constants are fitted to kernel-trace durations of the
// 64x64x64 tile on 30 grids of 16 to 361 tiles (K from 256 to 8192), each
// at S = 1, 2, 3, 4, 5, 6, 8, 12 and 16 (log residuals 6% rms); over those
// grids the chosen factor runs within 0.8% of the fastest measured one on
// average (17% at worst, 320^3).  SGEMM_SPLITK forces a factor (clamped to
// the K tiles and the workspace) for sweeps.
constexpr double kBlockFixed = 2.8;
constexpr double kSplitFixed = 1.7;
constexpr double kSplitPerPartial = 0.45;
double split_cost(long tiles, long kt, long s, int bm, int bn) {
    const long r = ceil_div(tiles * s, kNumCUs);
    const double busiest = (double)(r * ceil_div(kt, s)) + (double)ceil_div(r, 2) * kBlockFixed;
    const double floor = 0.15 * (double)(tiles * kt) * (double)(bm + bn) / ((double)bm * bn);
    const double partials = s > 1 ? kSplitFixed + kSplitPerPartial * (double)s : 0.0;
    return (busiest > floor ? busiest : floor) + partials;
}

// (`batch` problems of one strided batch count as batch times the tiles)
int choose_splits(int M, int N, int K, int bm, int bn, int bk, long batch = 1) {
    const long tiles = ceil_div(M, bm) * ceil_div(N, bn) * batch;
    const long kt = ceil_div(K, bk);
    const long fit = (long)(kSplitPartialBytes / ((size_t)bm * bn * sizeof(float)));
    if (tiles > kSplitMaxTiles || kt < 2) return 1;
    if (knobs().splitk > 0) {
        long s = knobs().splitk;
        if (s * tiles > fit) s = fit / tiles;
        if (s > kt) s = kt;
        return s < 1 ? 1 : (int)s;
    }
    if (tiles >= kTailSlots) return 1;
    const double base = split_cost(tiles, kt, 1, bm, bn);
    long best = 1;
    double best_cost = base;
    for (long s = 2; s <= 16 && s <= kt / 2 && s * tiles <= fit; ++s) {
        const double cost = split_cost(tiles, kt, s, bm, bn);
        if (cost < best_cost) {
            best = s;
            best_cost = cost;
        }
    }
    return best_cost <= 0.95 * base ? (int)best : 1;
}

// ---------------------------------------------------------------------------
// Device memory kept between calls.  Two kinds: split-K workspaces (partial
// tiles and tile counters, kSplitWorkspaceBytes each) and copy buffers (for
// operands copied before the product, grown on demand).  A device keeps at
// most SGEMM_MAX_STREAM_WORKSPACES workspaces and SGEMM_MAX_COPY_BUFFERS
// copy buffers, each bound to one stream (the per-thread default stream
// counts once per host thread).
//
// A call leases its stream's slot from before its first launch to after its
// last.  A stream without a slot gets a new one while the device has fewer
// than the maximum, else the least recently used slot that no call holds,
// once the kernels queued on it have finished: however many streams a
// process creates and destroys, the memory stays bounded, and a buffer is
// never handed to another stream while kernels that use it are queued.
//
// What marks a slot's last use: the end of a lease records an event on the
// stream.  A workspace skips that record while no stream of its device has
// ever found every workspace taken (the event's marker costs the queue
// about 3 us, as much as a small split saves): then no workspace is handed
// over, so none needs it.  The first stream to find them all taken sets the
// device "contended" for good, from which point every lease end records;
// idle workspaces whose last use went unrecorded are handed over only after
// one hipDeviceSynchronize, once.  Copy buffers record at every lease end.
// All waits (on an event, the one drain, or before a copy buffer grows)
// happen outside the lock, so a call never blocks calls on other streams.
//
// When no slot can be had without waiting for another call (every slot of
// the device held), the call takes a path that needs none: K is not split,
// or the operand is not copied.  Nothing is allocated, cleared or waited
// for under graph capture; such calls take those paths too.
//
// Workspaces may be shared by calls on one stream, which run in stream
// order; a copy buffer is held by one call at a time (its copies and the
// product that reads them are separate launches).
enum SlotKind { kWorkspaceSlot = 0, kCopySlot = 1 };
constexpr int kUnavailable = 1;          // acquire(): no slot without waiting

// How a slot's last use is known to be over.
enum LastUse {
    kNoUse = 0,                          // new or drained: nothing queued uses it
    kEventMarks = 1,                     // `done` was recorded after the last lease
    kUnmarked = 2,                       // a lease ended without a record: only its own stream may use it
};

struct Slot {
    int kind = 0;
    int dev = -1;
    hipStream_t stream = nullptr;
    std::thread::id thread;              // the host thread, for hipStreamPerThread
    void *mem = nullptr;
    size_t bytes = 0;
    hipEvent_t done = nullptr;           // recorded at the end of a lease (see LastUse)
    int last_use = kNoUse;
    int users = 0;                       // calls holding a lease
    bool moving = false;                 // being set up, grown or handed over (unlocked)
    bool pinned = false;                 // an event record failed: never handed over
    unsigned long long stamp = 0;        // last use, for least-recently-used choice
};

struct Lease {
    Slot *slot = nullptr;
    void *mem = nullptr;
};

std::mutex g_slot_mu;
std::list<Slot> g_slots;                 // node addresses stay valid
unsigned long long g_slot_clock = 0;
std::vector<int> g_contended;            // devices where a stream found every workspace taken (never cleared)

int max_slots(int kind) { return kind == kWorkspaceSlot ? SGEMM_MAX_STREAM_WORKSPACES : SGEMM_MAX_COPY_BUFFERS; }

bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &cap) == hipSuccess && cap != hipStreamCaptureStatusNone;
}

bool contended(int dev) {
    return std::find(g_contended.begin(), g_contended.end(), dev) != g_contended.end();
}

// (Unlocked; the slot is marked moving.)  Make `s` hold at least `bytes`
// for `stream`: wait for its last use, replace memory that is too small, and
// clear a workspace's tile counters on the stream.
int prepare_slot(Slot &s, size_t bytes, hipStream_t stream) {
    hipError_t e = hipSuccess;
    if (s.done == nullptr) {
        e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
        if (e != hipSuccess) {
            s.done = nullptr;
            return record_hip_error(e, "hipEventCreateWithFlags");
        }
    }
    if (s.last_use == kUnmarked) {
        // only the slot's own stream gets here (acquire_slot hands over no
        // unmarked slot): the kernels queued on it include the last use
        e = hipEventRecord(s.done, stream);
        if (e != hipSuccess) return record_hip_error(e, "hipEventRecord (buffer growth)");
        s.last_use = kEventMarks;
    }
    if (s.last_use == kEventMarks) {
        e = hipEventSynchronize(s.done);
        if (e != hipSuccess) return record_hip_error(e, "hipEventSynchronize (buffer hand-over)");
        s.last_use = kNoUse;
    }
    if (s.mem == nullptr || s.bytes < bytes) {
        if (s.mem != nullptr) {
            e = hipFree(s.mem);
            s.mem = nullptr;
            s.bytes = 0;
            if (e != hipSuccess) return record_hip_error(e, "hipFree (buffer)");
        }
        e = hipMalloc(&s.mem, bytes);
        if (e != hipSuccess) {
            s.mem = nullptr;
            return record_hip_error(e, s.kind == kWorkspaceSlot ? "hipMalloc (split-K workspace)"
                                                               : "hipMalloc (copy buffer)");
        }
        s.bytes = bytes;
    }
    if (s.kind == kWorkspaceSlot) {
        e = hipMemsetAsync(static_cast<char *>(s.mem) + kSplitPartialBytes, 0, kSplitMaxTiles * sizeof(unsigned),
                           stream);
        if (e != hipSuccess) return record_hip_error(e, "hipMemsetAsync (split-K counters)");
    }
    return SGEMM_STATUS_OK;
}

// Lease the slot of `kind` for `stream` with at least `bytes`: returns
// SGEMM_STATUS_OK (out.mem set), kUnavailable (take a path without the
// buffer) or an error status.
int acquire_slot(int kind, hipStream_t stream, size_t bytes, Lease &out) {
    out = Lease{};
    if (capturing(stream)) return kUnavailable;
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record_hip_error(e, "hipGetDevice");
    const std::thread::id thread = stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
    std::unique_lock<std::mutex> lock(g_slot_mu);
    Slot *s = nullptr;
    for (bool drained = false;;) {
        Slot *lru = nullptr;
        std::vector<Slot *> unmarked;
        int held = 0;
        s = nullptr;
        for (Slot &x : g_slots) {
            if (x.kind != kind || x.dev != dev) continue;
            ++held;
            if (x.stream == stream && x.thread == thread) s = &x;
            if (x.users != 0 || x.moving || x.pinned) continue;
            if (x.last_use == kUnmarked) {
                unmarked.push_back(&x);
            } else if (lru == nullptr || x.stamp < lru->stamp) {
                lru = &x;
            }
        }
        if (s != nullptr) {
            if (s->moving || (kind == kCopySlot && s->users > 0) || s->pinned) return kUnavailable;
            if (s->bytes >= bytes) {
                ++s->users;
                s->stamp = ++g_slot_clock;
                out = Lease{s, s->mem};
                return SGEMM_STATUS_OK;
            }
            if (s->users > 0) return kUnavailable;         // grow only while no call holds it
            break;
        }
        if (held < max_slots(kind)) {
            g_slots.emplace_back();
            s = &g_slots.back();
            s->kind = kind;
            s->dev = dev;
            break;
        }
        if (kind == kWorkspaceSlot && !contended(dev)) g_contended.push_back(dev);   // lease ends record from now on
        if (lru != nullptr) {
            s = lru;
            break;
        }
        if (unmarked.empty() || drained) return kUnavailable;
        // Idle workspaces whose last use went unrecorded: wait once for the
        // device to drain (outside the lock), after which they hold nothing
        // queued.  A failed wait leaves them as they were and this call
        // unsplit.
        for (Slot *x : unmarked) x->moving = true;
        lock.unlock();
        const hipError_t se = hipDeviceSynchronize();
        lock.lock();
        for (Slot *x : unmarked) {
            x->moving = false;
            if (se == hipSuccess && x->last_use == kUnmarked) x->last_use = kNoUse;
        }
        if (se != hipSuccess) return kUnavailable;
        drained = true;
    }
    s->stream = stream;
    s->thread = thread;
    s->moving = true;
    lock.unlock();
    const int st = prepare_slot(*s, bytes, stream);
    lock.lock();
    s->moving = false;
    s->stamp = ++g_slot_clock;
    if (st != SGEMM_STATUS_OK) return st;
    ++s->users;
    out = Lease{s, s->mem};
    return SGEMM_STATUS_OK;
}

// End a lease: the slot's event marks this call's last use on `stream`
// (a workspace of a device never contended: left unmarked, see LastUse).
// Returns SGEMM_STATUS_OK or, if the event cannot be recorded, the HIP error
// (the slot is then never handed over or released).
int release_slot(Lease &l, hipStream_t stream) {
    if (l.slot == nullptr) return SGEMM_STATUS_OK;
    Slot *s = l.slot;
    l = Lease{};
    std::lock_guard<std::mutex> lock(g_slot_mu);
    --s->users;
    s->stamp = ++g_slot_clock;
    if (s->kind == kWorkspaceSlot && !contended(s->dev)) {
        s->last_use = kUnmarked;
        return SGEMM_STATUS_OK;
    }
    const hipError_t e = hipEventRecord(s->done, stream);
    if (e != hipSuccess) {
        s->pinned = true;
        return record_hip_error(e, "hipEventRecord (buffer release)");
    }
    s->last_use = kEventMarks;
    return SGEMM_STATUS_OK;
}

// Split K `splits` ways (when above one) with the stream's workspace: sets
// a.splits, a.ws and a.counters and the lease; leaves a.splits at 1 when
// no workspace is available (graph capture, every workspace held).
int attach_workspace(Args &a, int splits, hipStream_t stream, Lease &lease) {
    if (splits <= 1) return SGEMM_STATUS_OK;
    if (lease.slot == nullptr) {
        const int st = acquire_slot(kWorkspaceSlot, stream, kSplitWorkspaceBytes, lease);
        if (st == kUnavailable) return SGEMM_STATUS_OK;
        if (st != SGEMM_STATUS_OK) return st;
    }
    a.splits = splits;
    a.ws = static_cast<float *>(lease.mem);
    a.counters = reinterpret_cast<unsigned *>(static_cast<char *>(lease.mem) + kSplitPartialBytes);
    return SGEMM_STATUS_OK;
}

// The first error of a call's launches and its lease's release.
int finish(hipError_t launch, Lease &lease, hipStream_t stream) {
    const int rel = release_slot(lease, stream);
    if (launch != hipSuccess) return record_hip_error(launch, "kernel launch");
    return rel;
}

// ---------------------------------------------------------------------------
// Scratch of sgemm_noalloc(), for callers that cannot allocate: the split-K
// partial tiles and tile counters of a call live in this file-scope device
// array, which exists from the moment the library's code is loaded on a
// device until the process ends (one copy per device).  Its device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept; host code uses only that address, never the array's
// name, which on the host is a stand-in without device meaning.  The
// counters a call uses are cleared by a small kernel on the call's stream
// before the product (no hipMemsetAsync, so the calls can be captured into
// a graph).  Every call on a device shares the array: calls that overlap
// in time on one device race.
// As large as a split-K workspace: the planner keeps every split, forced
// factors included, within kSplitPartialBytes (128x128 last-wave splits of
// the automatic choice reach 63 MiB), so each plan sgemm() makes fits.
constexpr size_t kScratchPartialBytes = kSplitPartialBytes;
constexpr size_t kScratchBytes = kScratchPartialBytes + kSplitMaxTiles * sizeof(unsigned);
static_assert(kScratchBytes == (size_t)SGEMM_NOALLOC_SCRATCH_BYTES, "scratch size in sgemm.h");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<std::pair<int, void *>> g_scratch_ptr;   // (device, address of `scratch` there)

// The device address of this device's `scratch`.
int scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record_hip_error(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    for (const auto &x : g_scratch_ptr)
        if (x.first == dev) {
            *out = x.second;
            return SGEMM_STATUS_OK;
        }
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
        return record_hip_error(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress (scratch)");
    g_scratch_ptr.emplace_back(dev, ptr);
    *out = ptr;
    return SGEMM_STATUS_OK;
}

__global__ void __launch_bounds__(256) clear_counters_kernel(unsigned *counters, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) counters[i] = 0u;
}

// Split K `splits` ways over the launch's `tiles` tiles in the scratch at
// `ptr`: clears the counters on the stream and sets a.splits, a.ws and
// a.counters.  The caller has checked that the partials fit.
hipError_t attach_scratch(Args &a, int splits, long tiles, void *ptr, hipStream_t stream) {
    a.splits = splits;
    a.ws = static_cast<float *>(ptr);
    a.counters = reinterpret_cast<unsigned *>(static_cast<char *>(ptr) + kScratchPartialBytes);
    return launch_k(clear_counters_kernel, dim3((unsigned)ceil_div(tiles, 256)), dim3(256), stream, a.counters,
                    (int)tiles);
}

// Wave quantization: a grid of whole waves plus a partly filled last wave
// can run as two launches, the whole waves as they are and the last wave
// with K split S ways, so that the last wave's few tiles spread over the
// whole chip.  Workgroup slots: two per compute unit (kTailSlots).  Cost of
// the last wave in the K-tile steps of split_cost: unsplit, its `rem` tiles
// run one per CU, kt + kTailBlockFixed steps; split S ways,
// ceil(rem * S / 256) blocks of ceil(kt / S) + kTailBlockFixed steps on the
// busiest CU, plus the partials' traffic (0.49 * S * rem / bk steps: 8 * S
// * bm * bn bytes per tile at about 5 TB/s) and a fixed kTailFixed for the
// second launch
// and the hand-off.  S (at most 16, at least three K tiles per split, within
// the workspace) is the factor of least cost, taken when it costs at most
// 95% of the unsplit last wave; 1 = one launch.  kTailFixed is fitted to the
// split and unsplit 64x64x64 kernel timed side by side with the earlier rule
// of splitting every last wave up to a quarter full (1536^3 +4%,
// 2560x2624x2560 +2%, 1600^3 level, 1552x1572x1000 -7%, and 2944^2 x 256 on
// 64x64x32 tiles -16%): 4.5 to 13 steps, 8 taken, which splits the first
// two and neither of the last two.  SGEMM_TAIL_FILL (percent) caps the fill
// of a last wave that may be split, for sweeps.
struct VariantDesc;
int choose_tail_splits(const VariantDesc &d, const Args &a);

// A split-capable variant: split-K when a.splits > 1, else the plain lean
// kernel of the same tile.
typedef hipError_t (*SplitLauncher)(const Args &, int, hipStream_t);
template <SplitLauncher SPLIT, Launcher PLAIN>
hipError_t launch_split_or_plain(const Args &a, hipStream_t stream) {
    return a.splits > 1 ? SPLIT(a, a.splits, stream) : PLAIN(a, stream);
}

// Whether the byte offsets within one K tile of the lean kernel's part of A
// and B fit the buffer descriptors' 31-bit range (the operands themselves
// may be larger: every tile gets its own descriptor base).
bool lean_fits(int bm, int bn, int bk, long lda, long ldb, bool ta, bool tb) {
    const long lim = 0x7fffffffL;
    const long spanA = ta ? (long)bk * lda + bm : (long)bm * lda + bk;
    const long spanB = tb ? (long)bn * ldb + bk : (long)bk * ldb + bn;
    return 4L * spanA < lim && 4L * spanB < lim;
}

// Whether the lean kernel of a bm x bn x bk tile takes the operands of an
// untransposed problem (else launch_lean_or runs its guarded fallback).
bool lean_takes(int bm, int bn, int bk, const Args &a) {
    return a.K >= bk && !(a.K % 4) && !(a.N % 4) && lean_fits(bm, bn, bk, a.lda, a.ldb, false, false);
}
// The same for the lean kernel with 4-byte loads (any K, N and alignment).
bool lean_dw_takes(int bm, int bn, int bk, const Args &a) {
    return a.K >= bk && lean_fits(bm, bn, bk, a.lda, a.ldb, false, false);
}

// The lean kernel takes K >= BK, K and N multiples of 4 (M, N and K need not
// be whole tiles) and offsets within a tile that fit the descriptors' range;
// other shapes go to FALLBACK, a guarded kernel.
template <int BM, int BN, int BK, Launcher LEAN, Launcher FALLBACK>
hipError_t launch_lean_or(const Args &a, hipStream_t stream) {
    // (a launch over part of the grid, a.tile_count > 0, is made only for
    // operands the lean kernel takes; the fallback always covers the whole
    // grid)
    if (lean_takes(BM, BN, BK, a)) return LEAN(a, stream);
    Args whole = a;
    whole.tile_base = whole.tile_count = 0;
    return FALLBACK(whole, stream);
}

// The lean kernel with 4-byte loads takes any alignment and any K >= BK, with
// offsets within a tile that fit as above; other shapes go to FALLBACK.
template <int BM, int BN, int BK, Launcher LEAN, Launcher FALLBACK>
hipError_t launch_lean_dw_or(const Args &a, hipStream_t stream) {
    if (lean_dw_takes(BM, BN, BK, a)) return LEAN(a, stream);
    Args whole = a;                      // the fallback covers the whole grid
    whole.tile_base = whole.tile_count = 0;
    return FALLBACK(whole, stream);
}

hipError_t launch_simple_general(const Args &a0, bool ta, bool tb, int batch, hipStream_t stream) {
    const Args a = tiled(a0, 64, 64);
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)batch), block(256);
    if (ta && tb) return launch_k(sgemm_simple_kernel<true, true>, grid, block, stream, a);
    if (ta) return launch_k(sgemm_simple_kernel<true, false>, grid, block, stream, a);
    if (tb) return launch_k(sgemm_simple_kernel<false, true>, grid, block, stream, a);
    return launch_k(sgemm_simple_kernel<false, false>, grid, block, stream, a);
}

hipError_t launch_simple(const Args &a, hipStream_t stream) { return launch_simple_general(a, false, false, 1, stream); }

// The plain kernel on 16-bit inputs (each element widened to FP32 on load).
hipError_t launch_simple_lowp(const Args &a0, bool f16, bool ta, bool tb, int batch, hipStream_t stream) {
    const Args a = tiled(a0, 64, 64);
    const dim3 grid((unsigned)(a.tiles_m * a.tiles_n), 1, (unsigned)batch), block(256);
#define SGEMM_S(A, B)                                                             \
    (f16 ? launch_k(sgemm_simple_kernel<A, B, kF16>, grid, block, stream, a)      \
         : launch_k(sgemm_simple_kernel<A, B, kBF16>, grid, block, stream, a))
    if (ta && tb) return SGEMM_S(true, true);
    if (ta) return SGEMM_S(true, false);
    if (tb) return SGEMM_S(false, true);
    return SGEMM_S(false, false);
#undef SGEMM_S
}

struct VariantDesc {
    const char *name;
    int bm, bn, bk;
    bool needs_vec;
    Launcher launch;
    bool split_k = false;   // may split K (needs the workspace)
    bool dw = false;        // lean kernel with 4-byte loads (any alignment)
};

// Ids 0..2 are the stable ones named in sgemm.h; the rest are tile shapes
// kept for sweeps (128-bit access only).
constexpr VariantDesc kVariants[] = {
    {"simple_64x64x16", 64, 64, 16, false, launch_simple},
    {"db_128x128x32_w2x2_vec", 128, 128, 32, true, launch_db<128, 128, 32, 2, 2, true>},
    {"db_128x128x32_w2x2_scalar", 128, 128, 32, false, launch_db<128, 128, 32, 2, 2, false>},
    {"db_128x128x16_w2x2_vec", 128, 128, 16, true, launch_db<128, 128, 16, 2, 2, true>},
    {"db_128x128x64_w2x2_vec", 128, 128, 64, true, launch_db<128, 128, 64, 2, 2, true>},
    {"db_256x128x32_w4x2_vec", 256, 128, 32, true, launch_db<256, 128, 32, 4, 2, true>},
    {"db_128x256x32_w2x4_vec", 128, 256, 32, true, launch_db<128, 256, 32, 2, 4, true>},
    {"db_256x128x32_w2x2_vec", 256, 128, 32, true, launch_db<256, 128, 32, 2, 2, true>},
    {"db_128x256x32_w2x2_vec", 128, 256, 32, true, launch_db<128, 256, 32, 2, 2, true>},
    {"db_256x256x32_w2x2_vec", 256, 256, 32, true, launch_db<256, 256, 32, 2, 2, true>},
    {"db_256x256x32_w4x2_vec", 256, 256, 32, true, launch_db<256, 256, 32, 4, 2, true>},
    {"db_256x256x16_w4x4_vec", 256, 256, 16, true, launch_db<256, 256, 16, 4, 4, true>},
    {"db_256x128x16_w4x2_vec", 256, 128, 16, true, launch_db<256, 128, 16, 4, 2, true>},
    {"db_256x256x16_w2x4_vec", 256, 256, 16, true, launch_db<256, 256, 16, 2, 4, true>},
    {"pipe_256x128x16_w2x2_vec", 256, 128, 16, true, launch_pipe<256, 128, 2, 2, true>},
    {"pipe_128x128x16_w2x2_vec", 128, 128, 16, true, launch_pipe<128, 128, 2, 2, true>},
    {"sec_128x128x64_w2x2_vec", 128, 128, 64, true, launch_sec<128, 128, 64, 2, 2, true>},
    {"sec_128x128x32_w2x2_vec", 128, 128, 32, true, launch_sec<128, 128, 32, 2, 2, true>},
    {"sec_256x128x32_w2x2_vec", 256, 128, 32, true, launch_sec<256, 128, 32, 2, 2, true>},
    {"sec_128x256x32_w2x2_vec", 128, 256, 32, true, launch_sec<128, 256, 32, 2, 2, true>},
    {"dtl_128x128x64_w2x2_s2", 128, 128, 64, true, launch_dtl<128, 128, 64, 2, 2, 2>},
    {"dtl_128x128x32_w2x2_s3", 128, 128, 32, true, launch_dtl<128, 128, 32, 2, 2, 3>},
    {"dtl_256x128x32_w2x2_s3", 256, 128, 32, true, launch_dtl<256, 128, 32, 2, 2, 3>},
    {"lean_128x128x64_w2x2", 128, 128, 64, true,
     launch_lean_or<128, 128, 64, launch_lean_128x128x64_w2x2, launch_sec<128, 128, 64, 2, 2, true>>},
    {"lean_128x128x32_w2x2", 128, 128, 32, true,
     launch_lean_or<128, 128, 32, launch_lean_128x128x32_w2x2, launch_sec<128, 128, 32, 2, 2, true>>},
    {"lean_256x128x32_w4x2", 256, 128, 32, true,
     launch_lean_or<256, 128, 32, launch_lean_256x128x32_w4x2, launch_db<256, 128, 32, 4, 2, true>>},
    {"lean_128x256x32_w2x4", 128, 256, 32, true,
     launch_lean_or<128, 256, 32, launch_lean_128x256x32_w2x4, launch_db<128, 256, 32, 2, 4, true>>},
    {"lean_128x128x32_w2x2_splitk", 128, 128, 32, true,
     launch_lean_or<128, 128, 32,
                    launch_split_or_plain<launch_lean_splitk_128x128x32_w2x2, launch_lean_128x128x32_w2x2>,
                    launch_sec<128, 128, 32, 2, 2, true>>,
     true},
    // smaller tiles for small problems (guarded fallback: the 128x128x32
    // section-pipelined kernel)
    {"lean_64x64x32_w4x1", 64, 64, 32, true,
     launch_lean_or<64, 64, 32, launch_lean_64x64x32_w4x1, launch_sec<128, 128, 32, 2, 2, true>>},
    {"lean_64x64x32_w4x1_splitk", 64, 64, 32, true,
     launch_lean_or<64, 64, 32, launch_split_or_plain<launch_lean_splitk_64x64x32_w4x1, launch_lean_64x64x32_w4x1>,
                    launch_sec<128, 128, 32, 2, 2, true>>,
     true},
    {"lean_64x64x64_w4x1", 64, 64, 64, true,
     launch_lean_or<64, 64, 64, launch_lean_64x64x64_w4x1, launch_sec<128, 128, 32, 2, 2, true>>},
    {"lean_64x64x64_w4x1_splitk", 64, 64, 64, true,
     launch_lean_or<64, 64, 64, launch_split_or_plain<launch_lean_splitk_64x64x64_w4x1, launch_lean_64x64x64_w4x1>,
                    launch_sec<128, 128, 32, 2, 2, true>>,
     true},
    {"lean_64x128x32_w2x2", 64, 128, 32, true,
     launch_lean_or<64, 128, 32, launch_lean_64x128x32_w2x2, launch_sec<128, 128, 32, 2, 2, true>>},
    {"lean_64x128x32_w2x2_splitk", 64, 128, 32, true,
     launch_lean_or<64, 128, 32, launch_split_or_plain<launch_lean_splitk_64x128x32_w2x2, launch_lean_64x128x32_w2x2>,
                    launch_sec<128, 128, 32, 2, 2, true>>,
     true},
    {"lean_128x64x32_w4x1", 128, 64, 32, true,
     launch_lean_or<128, 64, 32, launch_lean_128x64x32_w4x1, launch_sec<128, 128, 32, 2, 2, true>>},
    {"lean_128x64x32_w4x1_splitk", 128, 64, 32, true,
     launch_lean_or<128, 64, 32, launch_split_or_plain<launch_lean_splitk_128x64x32_w4x1, launch_lean_128x64x32_w4x1>,
                    launch_sec<128, 128, 32, 2, 2, true>>,
     true},
    // any alignment (4-byte direct loads; guarded fallback: the 32-bit
    // double-buffered kernel)
    {"lean_dw_128x128x32_w2x2", 128, 128, 32, false,
     launch_lean_dw_or<128, 128, 32, launch_lean_dw_128x128x32_w2x2, launch_db<128, 128, 32, 2, 2, false>>},
    {"lean_dw_64x64x64_w4x1", 64, 64, 64, false,
     launch_lean_dw_or<64, 64, 64, launch_lean_dw_64x64x64_w4x1, launch_db<128, 128, 32, 2, 2, false>>},
    {"lean_dw_64x64x64_w4x1_splitk", 64, 64, 64, false,
     launch_lean_dw_or<64, 64, 64,
                       launch_split_or_plain<launch_lean_splitk_dw_64x64x64_w4x1, launch_lean_dw_64x64x64_w4x1>,
                       launch_db<128, 128, 32, 2, 2, false>>,
     true, true},
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

constexpr double kTailFixed = 8.0;
constexpr double kTailBlockFixed = 3.0;
// The last-wave split factor of an M x N x K grid of bm x bn x bk tiles.
int tail_split_factor(int M, int N, int K, int bm, int bn, int bk) {
    const long tiles = ceil_div(M, bm) * ceil_div(N, bn);
    const long rem = tiles % kTailSlots;
    if (tiles < kTailSlots || rem == 0 || rem * 100 > kTailSlots * knobs().tail_fill || rem > kSplitMaxTiles)
        return 1;
    const long kt = ceil_div(K, bk);
    const long fit = (long)(kSplitPartialBytes / ((size_t)bm * bn * sizeof(float) * rem));
    const double base = (double)ceil_div(rem, kNumCUs) * ((double)kt + kTailBlockFixed);
    long best = 1;
    double best_cost = base;
    for (long s = 2; s <= 16 && s <= kt / 3 && s <= fit; ++s) {
        const double cost = (double)ceil_div(rem * s, kNumCUs) * ((double)ceil_div(kt, s) + kTailBlockFixed) +
                            0.49 * (double)(s * rem) / bk + kTailFixed;
        if (cost < best_cost) {
            best = s;
            best_cost = cost;
        }
    }
    return best_cost <= 0.95 * base ? (int)best : 1;
}

int choose_tail_splits(const VariantDesc &d, const Args &a) {
    if (!(d.dw ? lean_dw_takes(d.bm, d.bn, d.bk, a) : lean_takes(d.bm, d.bn, d.bk, a))) return 1;
    return tail_split_factor(a.M, a.N, a.K, d.bm, d.bn, d.bk);
}

// Variants the automatic choice uses (indices into kVariants, looked up by
// name at compile time).
constexpr bool same_name(const char *x, const char *y) {
    while (*x != 0 && *x == *y) {
        ++x;
        ++y;
    }
    return *x == *y;
}
constexpr int variant_id(const char *name) {
    for (int i = 0; i < kNumVariants; ++i)
        if (same_name(kVariants[i].name, name)) return i;
    return -1;
}
// (the 128x128x32 form the automatic choice takes is the split-capable one:
// on whole waves it launches the plain kernel, and a partly filled last wave
// of tiles is split as for 64x64x64 tiles: 6000^3 to 7744^3 1.8-3.2% faster)
constexpr int kVec = variant_id("lean_128x128x32_w2x2_splitk");
constexpr int kVec64 = variant_id("lean_64x64x64_w4x1_splitk");
constexpr int kVec64ShortK = variant_id("lean_64x64x32_w4x1_splitk");
constexpr int kAny = variant_id("lean_dw_128x128x32_w2x2");          // 4-byte loads, any alignment
constexpr int kAny64 = variant_id("lean_dw_64x64x64_w4x1_splitk");
static_assert(kVec >= 0 && kVec64 >= 0 && kVec64ShortK >= 0 && kAny >= 0 && kAny64 >= 0, "variant table");
constexpr int kMaxBatch = 65535;  // problems per strided batch (launch grid z extent)

// Fill of the last wave of blocks: with t tiles spread over the CUs, the
// busiest CU runs ceil(t / 256) tiles while the average is t / 256.
double wave_fill(long tiles) {
    const long rounds = ceil_div(tiles, kNumCUs);
    return rounds > 0 ? (double)tiles / (double)(rounds * kNumCUs) : 0.0;
}

// Tile choice of the automatic dispatch: the 64x64 tile when the 128x128
// grid has at most 256 tiles (both kernels run two workgroups per compute
// unit, so such a grid leaves half the slots empty), or when the last wave
// of 64x64 tiles is fuller by more than the 3% that the smaller tile costs
// in throughput at full occupancy.  Measured (bench.py --sweep): 64x64x64
// ahead at 768^3 to 3584^3 and 5120^3, 128x128x32 ahead at 4096^3, 8192^3
// and short K.  (`batch` problems of one strided batch count as batch times
// the tiles)
bool prefer_64(int M, int N, long batch = 1) {
    const long t128 = ceil_div(M, 128) * ceil_div(N, 128) * batch;
    const long t64 = ceil_div(M, 64) * ceil_div(N, 64) * batch;
    return t128 <= kNumCUs || wave_fill(t64) * 0.97 > wave_fill(t128);
}

// Automatic choice: the lean kernel with 16-byte loads when the operands
// allow them, else the lean kernel with 4-byte loads; the tile by
// prefer_64(); the split-capable forms split K where choose_splits() or
// choose_tail_splits() says so.  Short K (at most 256) on a grid of at
// least one full wave of 64x64 tiles takes the 32-deep K tile, whose
// shorter first loads and pipeline fill weigh less over few K tiles:
// 1536^2, 1600^2, 2048^2, 2560x2624 and 2944^2 at K = 128 and 256 2-9%
// faster than the 64-deep one (at K = 384 and 512 the two trade places
// with the shape, at K = 1024 the 64-deep one leads by 8%; with at most 8
// K tiles of 32 no last-wave split pays).  No HIP call.
int auto_variant(int M, int N, int K, const float *A, int lda, const float *B, int ldb, float beta,
                 const float *C, int ldc) {
    const bool small = prefer_64(M, N);
    // (the 16-byte kernels also need K and N multiples of 4: whole chunks
    // at the edges; aligned operands with other K or N take the 4-byte ones)
    if (!vec_ok(K, A, lda, B, ldb, beta, C, ldc) || K % 4 || N % 4) return small ? kAny64 : kAny;
    if (small && K <= 256 && ceil_div(M, 64) * ceil_div(N, 64) >= kTailSlots) return kVec64ShortK;
    return small ? kVec64 : kVec;
}

// noalloc: split-K partials and counters in `scratch` (sgemm_noalloc), the
// same plan as with the library's workspaces; a plan whose partials do not
// fit is refused with SGEMM_STATUS_SCRATCH_TOO_SMALL before any launch.
// The plan of run() with the split-K partials and counters in `scratch`:
// K split over the whole grid (choose_splits), or the last wave split
// (choose_tail_splits), or neither; nothing allocated.
int run_noalloc(const VariantDesc &d, Args a, hipStream_t s) {
    const long tiles = (long)a.tiles_m * a.tiles_n, rem = tiles % kTailSlots;
    const size_t tile_bytes = (size_t)d.bm * d.bn * sizeof(float);
    const int splits = d.split_k ? choose_splits(a.M, a.N, a.K, d.bm, d.bn, d.bk) : 1;
    const int tail_splits = d.split_k && splits == 1 ? choose_tail_splits(d, a) : 1;
    const size_t need = splits > 1 ? (size_t)splits * tiles * tile_bytes
                                   : (tail_splits > 1 ? (size_t)tail_splits * rem * tile_bytes : 0);
    if (need > kScratchPartialBytes) return SGEMM_STATUS_SCRATCH_TOO_SMALL;
    if (need == 0) {
        const hipError_t e = d.launch(a, s);
        return e == hipSuccess ? SGEMM_STATUS_OK : record_hip_error(e, "kernel launch");
    }
    void *ptr = nullptr;
    const int st = scratch_address(&ptr);
    if (st != SGEMM_STATUS_OK) return st;
    hipError_t e = hipSuccess;
    if (splits > 1) {
        e = attach_scratch(a, splits, tiles, ptr, s);
        if (e == hipSuccess) e = d.launch(a, s);
    } else {
        // whole waves first, then the last wave with K split, as in run()
        Args head = a, tail = a;
        head.tile_count = (int)(tiles - rem);
        tail.tile_base = (int)(tiles - rem);
        tail.tile_count = (int)rem;
        e = attach_scratch(tail, tail_splits, rem, ptr, s);
        if (e == hipSuccess) e = d.launch(head, s);
        if (e == hipSuccess) e = d.launch(tail, s);
    }
    return e == hipSuccess ? SGEMM_STATUS_OK : record_hip_error(e, "kernel launch");
}

int run(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
        float beta, float *C, int ldc, void *stream, int variant, bool noalloc = false) {
    int st = check_args(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_STATUS_OK) return st;
    if (variant < SGEMM_VARIANT_AUTO || variant >= kNumVariants) return SGEMM_STATUS_INVALID_VARIANT;
    if (M == 0 || N == 0) return SGEMM_STATUS_OK;
    if (variant == SGEMM_VARIANT_AUTO) variant = auto_variant(M, N, K, A, lda, B, ldb, beta, C, ldc);
    const VariantDesc &d = kVariants[variant];
    if (d.needs_vec && !vec_ok(K, A, lda, B, ldb, beta, C, ldc)) return SGEMM_STATUS_UNSUPPORTED;

    const long tiles_m = ceil_div(M, d.bm), tiles_n = ceil_div(N, d.bn);
    if (tiles_m * tiles_n > 0x7fffffffL) return SGEMM_STATUS_INVALID_DIM;

    Args a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = M;
    a.N = N;
    a.K = K;
    a.alpha = alpha;
    a.beta = beta;
    a.tiles_m = (int)tiles_m;
    a.tiles_n = (int)tiles_n;
    a.group_m = knobs().group_m;
    a.xcd_remap = knobs().xcd_remap;
    a.splits = 1;
    a.tile_base = a.tile_count = 0;
    a.ws = nullptr;
    a.counters = nullptr;
    a.strideA = a.strideB = a.strideC = 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (noalloc) return run_noalloc(d, a, s);
    Lease lease;
    if (d.split_k) {
        const int ws = attach_workspace(a, choose_splits(M, N, K, d.bm, d.bn, d.bk), s, lease);
        if (ws != SGEMM_STATUS_OK) return ws;
    }
    const int tail_splits = d.split_k && a.splits == 1 ? choose_tail_splits(d, a) : 1;
    if (tail_splits > 1) {
        // Whole waves of tiles first, then the last, partly filled wave with
        // K split: two launches on the stream, over disjoint tiles of C.
        const long tiles = tiles_m * tiles_n, rem = tiles % kTailSlots;
        Args head = a, tail = a;
        head.tile_count = (int)(tiles - rem);
        tail.tile_base = (int)(tiles - rem);
        tail.tile_count = (int)rem;
        const int ws = attach_workspace(tail, tail_splits, s, lease);
        if (ws != SGEMM_STATUS_OK) return ws;
        if (tail.splits > 1) {
            hipError_t e = d.launch(head, s);
            if (e == hipSuccess) e = d.launch(tail, s);
            return finish(e, lease, s);
        }
    }
    return finish(d.launch(a, s), lease, s);
}

// Transposed operands and strided batches (row-major).  op_a / op_b are
// SGEMM_OP_N or SGEMM_OP_T; A is M x K (stored K x M when transposed), B is
// K x N (stored N x K when transposed).  An untransposed single problem takes
// run() and its automatic choice.  Otherwise: the lean kernel (16-byte loads
// for untransposed aligned operands, else 4-byte loads) on the tile
// prefer_64() picks for batch x tiles; on 64x64x64 tiles with 16-byte
// loads K splits as in run(): over the whole grid (a batch's tiles counted
// together) or, for one problem, over the last wave; the other forms do not
// split; shapes the lean kernel does not take go to the plain kernel.
// ---------------------------------------------------------------------------
// Unaligned transposed operands.  A transposed operand without 16-byte rows
// takes the lean kernel's 4-byte gather, whose load instructions each touch
// up to 32 rows of the stored matrix: 45-71 TFLOP/s on 3001x4999x2048
// against about 125 untransposed.  (With 16-byte loads for the whole
// product, transposed operands run at the untransposed rate and stay as
// they are.)  For large enough problems, single or batched, the operand is
// instead transposed into a row-major copy (leading dimension rounded up to
// a multiple of 4, in a buffer of the library's) and the untransposed path
// runs on it.

// dst[c][r] = src[r][c] for r < rows, c < cols: 32x32 tiles through LDS (a
// padded row keeps the column reads conflict-free), both sides coalesced;
// problem z of a batch at src + z*src_stride and dst + z*dst_stride.
__global__ void __launch_bounds__(256) transpose_kernel(const float *__restrict__ src, long ld_src, int rows,
                                                        int cols, float *__restrict__ dst, long ld_dst,
                                                        long src_stride, long dst_stride) {
    __shared__ float t[32][33];
    const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    src += blockIdx.z * src_stride;
    dst += blockIdx.z * dst_stride;
#pragma unroll
    for (int i = ty; i < 32; i += 8) {
        const int r = r0 + i, c = c0 + tx;
        if (r < rows && c < cols) t[i][tx] = src[(long)r * ld_src + c];
    }
    __syncthreads();
#pragma unroll
    for (int i = ty; i < 32; i += 8) {
        const int c = c0 + i, r = r0 + tx;
        if (c < cols && r < rows) dst[(long)c * ld_dst + r] = t[tx][i];
    }
}

// Whether a transposed problem (or batch of `batch` problems, of which
// copies_a / copies_b distinct operands are copied) copies its unaligned
// transposed operands: not under graph capture (no allocation there), grid
// dimensions within the launch limits, copies within kCopyMaxBytes (the
// largest copy buffer, SGEMM_MAX_COPY_BUFFER_BYTES), and the
// copies' traffic (read and written once, at about 3 TB/s) taking less time
// than the product would at 120 TFLOP/s.
// Measured: the gather runs at 10-110 TFLOP/s (512^3 to 4095^3, 47-69 with
// both operands transposed), the copies and the untransposed kernel at
// 17-143, ahead at every size where this rule copies.
// SGEMM_PACK = 1 / -1 forces it on / off (where it can run).
constexpr double kCopyMaxBytes = (double)SGEMM_MAX_COPY_BUFFER_BYTES;

bool copy_plan(int M, int N, int K, bool copy_a, bool copy_b, void *stream, int batch = 1, int copies_a = 1,
               int copies_b = 1) {
    if (knobs().pack < 0 || (!copy_a && !copy_b)) return false;
    if (ceil_div(K, 32) > 65535 || ceil_div(copy_a ? M : N, 32) > 65535 || ceil_div(N, 32) > 65535) return false;
    const double copied = 4.0 * ((copy_a ? (double)copies_a * M * ((K + 3) & ~3L) : 0.0) +
                                 (copy_b ? (double)copies_b * K * ((N + 3) & ~3L) : 0.0));
    if (copied > kCopyMaxBytes) return false;
    if (capturing(reinterpret_cast<hipStream_t>(stream))) return false;
    if (knobs().pack > 0) return true;
    const double bytes = 8.0 * ((copy_a ? (double)copies_a * M * K : 0.0) + (copy_b ? (double)copies_b * K * N : 0.0));
    return bytes / 3e12 < 2.0 * batch * M * (double)N * K / 120e12;
}

int run_general(int op_a, int op_b, int M, int N, int K, float alpha, const float *A, int lda, long long sA,
                const float *B, int ldb, long long sB, float beta, float *C, int ldc, long long sC, int batch,
                void *stream);

// The product with the marked transposed operands replaced by row-major
// copies (A as M x K, B as K x N); an operand not copied keeps its form.  In
// a batch, an operand with stride 0 (one matrix for every problem) is copied
// once, and each other one per problem, 64-float aligned.  Returns
// kUnavailable, with nothing enqueued, when the stream's copy buffer is held
// by another call (the caller then gathers the operands instead).
int run_copied(int op_a, int op_b, bool copy_a, bool copy_b, int M, int N, int K, float alpha, const float *A,
               int lda, long long sA, const float *B, int ldb, long long sB, float beta, float *C, int ldc,
               long long sC, int batch, void *stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const long lda2 = (K + 3) & ~3L, ldb2 = (N + 3) & ~3L;
    const int na = batch > 1 && sA != 0 ? batch : 1, nb = batch > 1 && sB != 0 ? batch : 1;
    const size_t a_one = ((size_t)M * lda2 + 63) & ~(size_t)63, b_one = ((size_t)K * ldb2 + 63) & ~(size_t)63;
    const size_t a_floats = copy_a ? a_one * na : 0, b_floats = copy_b ? b_one * nb : 0;
    Lease lease;
    const int st = acquire_slot(kCopySlot, s, (a_floats + b_floats) * sizeof(float), lease);
    if (st != SGEMM_STATUS_OK) return st;
    float *buf = static_cast<float *>(lease.mem);
    hipError_t e = hipSuccess;
    if (copy_a) {   // stored K x M (leading dimension lda) -> M x K
        e = launch_k(transpose_kernel, dim3((unsigned)ceil_div(M, 32), (unsigned)ceil_div(K, 32), (unsigned)na),
                     dim3(256), s, A, (long)lda, K, M, buf, lda2, na > 1 ? (long)sA : 0L, (long)a_one);
        A = buf;
        lda = (int)lda2;
        sA = na > 1 ? (long long)a_one : 0;
    }
    if (copy_b && e == hipSuccess) {   // stored N x K (leading dimension ldb) -> K x N
        float *Bc = buf + a_floats;
        e = launch_k(transpose_kernel, dim3((unsigned)ceil_div(K, 32), (unsigned)ceil_div(N, 32), (unsigned)nb),
                     dim3(256), s, B, (long)ldb, N, K, Bc, ldb2, nb > 1 ? (long)sB : 0L, (long)b_one);
        B = Bc;
        ldb = (int)ldb2;
        sB = nb > 1 ? (long long)b_one : 0;
    }
    if (e != hipSuccess) return finish(e, lease, s);
    // (the copies are row-major and aligned, so this call copies nothing)
    const int prod = run_general(copy_a ? SGEMM_OP_N : op_a, copy_b ? SGEMM_OP_N : op_b, M, N, K, alpha, A, lda, sA,
                                 B, ldb, sB, beta, C, ldc, sC, batch, stream);
    const int rel = release_slot(lease, s);
    return prod != SGEMM_STATUS_OK ? prod : rel;
}

int run_general(int op_a, int op_b, int M, int N, int K, float alpha, const float *A, int lda, long long sA,
                const float *B, int ldb, long long sB, float beta, float *C, int ldc, long long sC, int batch,
                void *stream) {
    if ((op_a != SGEMM_OP_N && op_a != SGEMM_OP_T) || (op_b != SGEMM_OP_N && op_b != SGEMM_OP_T))
        return SGEMM_STATUS_INVALID_OP;
    const bool ta = op_a == SGEMM_OP_T, tb = op_b == SGEMM_OP_T;
    if (M < 0 || N < 0 || K < 0 || batch < 0 || batch > kMaxBatch) return SGEMM_STATUS_INVALID_DIM;
    const int need_lda = ta ? (M > 1 ? M : 1) : (K > 1 ? K : 1);
    const int need_ldb = tb ? (K > 1 ? K : 1) : (N > 1 ? N : 1);
    if (lda < need_lda || ldb < need_ldb || ldc < (N > 1 ? N : 1)) return SGEMM_STATUS_INVALID_DIM;
    if (batch > 1 && (sA < 0 || sB < 0 || (M > 0 && N > 0 && sC < (long long)(M - 1) * ldc + N)))
        return SGEMM_STATUS_INVALID_DIM;
    if (M == 0 || N == 0 || batch == 0) return SGEMM_STATUS_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return SGEMM_STATUS_NULL_POINTER;
    if (!ta && !tb && batch == 1)
        return run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, SGEMM_VARIANT_AUTO);
    if ((ta || tb) && K > 0) {
        // without 16-byte loads for the whole product (an operand or C
        // unaligned, an edge not in whole chunks, or a batch stride not a
        // multiple of 4) every transposed operand would be gathered
        const bool strides4 = batch == 1 || (sA % 4 == 0 && sB % 4 == 0 && sC % 4 == 0);
        const bool vec1 = strides4 && vec_ok(K, A, lda, B, ldb, beta, C, ldc) && (ta ? M : K) % 4 == 0 &&
                          (tb ? K : N) % 4 == 0;
        const bool copy_a = ta && !vec1, copy_b = tb && !vec1;
        const int na = batch > 1 && sA != 0 ? batch : 1, nb = batch > 1 && sB != 0 ? batch : 1;
        if (copy_plan(M, N, K, copy_a, copy_b, stream, batch, na, nb)) {
            const int st = run_copied(op_a, op_b, copy_a, copy_b, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C,
                                      ldc, sC, batch, stream);
            if (st != kUnavailable) return st;
        }
    }

    Args a;
    a.A = A;
    a.B = B;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = M;
    a.N = N;
    a.K = K;
    a.alpha = alpha;
    a.beta = beta;
    a.tiles_m = a.tiles_n = 0;   // set by each launcher from its tile
    a.group_m = knobs().group_m;
    a.xcd_remap = knobs().xcd_remap;
    a.splits = 1;
    a.tile_base = a.tile_count = 0;
    a.ws = nullptr;
    a.counters = nullptr;
    a.strideA = batch > 1 ? (long)sA : 0;
    a.strideB = batch > 1 ? (long)sB : 0;
    a.strideC = batch > 1 ? (long)sC : 0;

    // 16-byte loads: aligned operands with leading dimensions and strides
    // that are multiples of 4, and the edge chunks of each stored operand
    // whole (its contiguous extent a multiple of 4).
    const bool strides4 = batch == 1 || (sA % 4 == 0 && sB % 4 == 0 && sC % 4 == 0);
    const bool vec = strides4 && vec_ok(K, A, lda, B, ldb, beta, C, ldc) && (ta ? M : K) % 4 == 0 &&
                     (tb ? K : N) % 4 == 0;
    const bool tile64 = prefer_64(M, N, batch);
    const int bm = tile64 ? 64 : 128, bn = bm, bk = tile64 ? 64 : 32;
    const bool lean = K >= bk && lean_fits(bm, bn, bk, lda, ldb, ta, tb);

    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    if (lean && vec && tile64) {
        // 64x64x64 tiles with 16-byte loads: K split over the whole grid
        // (the tiles of every problem of a batch) or, for one problem, over
        // the last wave, by the cost models and with the workspaces of run().
        Lease lease;
        int ws = attach_workspace(a, choose_splits(M, N, K, 64, 64, 64, batch), s, lease);
        if (ws != SGEMM_STATUS_OK) return ws;
        if (a.splits > 1)
            return finish(launch_lean_splitk_g_64x64x64_w4x1(a, a.splits, ta, tb, batch, s), lease, s);
        const int tail_splits = batch == 1 ? tail_split_factor(M, N, K, 64, 64, 64) : 1;
        if (tail_splits > 1) {
            const long tiles = ceil_div(M, 64) * ceil_div(N, 64), rem = tiles % kTailSlots;
            Args head = a, tail = a;
            head.tile_count = (int)(tiles - rem);
            tail.tile_base = (int)(tiles - rem);
            tail.tile_count = (int)rem;
            ws = attach_workspace(tail, tail_splits, s, lease);
            if (ws != SGEMM_STATUS_OK) return ws;
            if (tail.splits > 1) {
                hipError_t e = launch_lean_general(head, true, false, ta, tb, 1, s);
                if (e == hipSuccess) e = launch_lean_splitk_g_64x64x64_w4x1(tail, tail.splits, ta, tb, 1, s);
                return finish(e, lease, s);
            }
        }
        return finish(launch_lean_general(a, true, false, ta, tb, batch, s), lease, s);
    }
    const hipError_t e =
        lean ? launch_lean_general(a, tile64, !vec, ta, tb, batch, s) : launch_simple_general(a, ta, tb, batch, s);
    if (e != hipSuccess) return record_hip_error(e, "kernel launch");
    return SGEMM_STATUS_OK;
}

// 16-bit inputs, FP32 accumulation and output.  Variant 0 is the plain
// kernel (any shape); the others are the direct-to-LDS kernel on a block
// tile and a number of LDS stages (`tile` of launch_lowp_tile = id - 1).
struct LowpVariant {
    const char *name;
    int bm, bn, bk;
};
const LowpVariant kLowpVariants[] = {
    {"lowp_simple_64x64", 64, 64, 16},
    {"lowp_128x128x64_s2", 128, 128, 64},
    {"lowp_256x128x64_s3", 256, 128, 64},
    {"lowp_256x256x32_s4", 256, 256, 32},
    {"lowp_256x256x32_s4_alt", 256, 256, 32},
    {"lowp_128x128x64_s4_alt", 128, 128, 64},
};
constexpr int kNumLowpVariants = (int)(sizeof(kLowpVariants) / sizeof(kLowpVariants[0]));

// Variants built for transposed operands: the two alternating kernels.
bool lowp_takes_ops(int variant) { return variant == 4 || variant == 5; }

// Whether the direct-to-LDS kernel of a bm x bn tile takes the operands: its
// loads are 16-byte chunks of 8 elements (aligned rows, N and K multiples of
// 8), K >= 64 keeps every K tile inside the operands (the remainder tile is
// taken first), and the buffer ranges of one block tile's part of a K tile
// fit in 31 bits.
// (ta / tb: A or B stored transposed.  A stored operand's contiguous extent,
// K for A and N for B, or M for A^T and K for B^T, must be whole chunks.)
bool lowp_fast_ok(const LowpVariant &v, int M, int N, int K, const void *A, int lda, const void *B, int ldb,
                  bool ta = false, bool tb = false) {
    const long lim = 0x7fffffffL;
    const long spanA = ta ? (long)v.bk * lda + v.bm : (long)v.bm * lda + v.bk;
    const long spanB = tb ? (long)v.bn * ldb + v.bk : (long)v.bk * ldb + v.bn;
    return aligned16(A) && aligned16(B) && lda % 8 == 0 && ldb % 8 == 0 && (ta ? M : K) % 8 == 0 &&
           (tb ? K : N) % 8 == 0 && K >= v.bk && 2L * spanA < lim && 2L * spanB < lim;
}

// The largest split-K factor a 16-bit kernel built with split-K may use:
// the 128x128 two-stage kernel and the 128x128 alternating kernel.  The tile
// grid must fill less than 3/4 of the kernel's workgroup slots (two per
// compute unit for the two-stage kernel, one for the alternating one), each
// split keeps at least eight K tiles, and the partial tiles fit the
// workspace.  1 for other variants.  Untransposed operands split on the
// alternating kernel from 16 tiles up only: below that its deeper pipeline
// fill costs more than it gains (BF16, split two-stage against split
// alternating: 128x128x2048 11.5 / 12.6 us, 256x256x4096 13.9 / 15.1,
// 384x256x8192 20.3 / 21.4; from 16 tiles the alternating one leads:
// 512x512x8192 25.3 / 24.2, 640x640x4096 20.5 / 18.6, 1024x1024x4096
// 24.9 / 20.7, 768x1024x16384 52.1 / 41.9).  Transposed operands (`ops`)
// have only the alternating kernels, and split on any grid.
// (`batch` problems of one strided batch count as batch times the tiles)
int lowp_max_splits(int variant, int M, int N, int K, long batch = 1, bool ops = false) {
    if (variant != 1 && variant != 5) return 1;
    const LowpVariant &v = kLowpVariants[variant];
    const long slots = variant == 1 ? 512 : 256;
    const long tiles = ceil_div(M, v.bm) * ceil_div(N, v.bn) * batch;
    if (variant == 5 && !ops && tiles < 16) return 1;
    if (tiles * 4 >= slots * 3 || tiles > kSplitMaxTiles) return 1;
    long s = slots / tiles;
    s = std::min(s, ceil_div(K, v.bk) / 8);
    s = std::min(s, 16L);
    s = std::min(s, (long)(kSplitPartialBytes / ((size_t)v.bm * v.bn * sizeof(float) * tiles)));
    return s < 1 ? 1 : (int)s;
}

// Predicted time (us) of a 16-bit variant with split factor s: waves of
// workgroups x (a workgroup's share of the product / its rate + 3 us of
// pipeline fill and epilogue), plus for s > 1 the partial tiles (written and
// read back, 2 s x M x N x 4 bytes at 5 TB/s) and 2 us.  Rates of one
// workgroup (TFLOP/s measured on MI355X): 2.07 for the 128x128 two-stage
// kernel with two per compute unit, 2.25 alone, 4.2 for the 256x128 kernel,
// 5.0 for the alternating 256x256 kernel and 3.3 for the alternating
// 128x128 kernel.
double lowp_predict_us(int variant, int s, int M, int N, int K, long batch = 1) {
    const LowpVariant &v = kLowpVariants[variant];
    const bool two_per_cu = variant == 1;
    const long blocks = ceil_div(M, v.bm) * ceil_div(N, v.bn) * s * batch;
    const double rate = variant == 1   ? (blocks <= 256 ? 2.25 : 2.07)
                        : variant == 2 ? 4.2
                        : variant == 5 ? 3.3
                                       : 5.0;
    const long waves = ceil_div(blocks, two_per_cu ? 512 : 256);
    double t = (double)waves * (2.0 * v.bm * v.bn * ((double)K / s) / (rate * 1e6) + 3.0);
    if (s > 1) t += 2.0 * s * (double)M * N * batch * 4 / 5e6 + 2.0;
    return t;
}

// The split factor of a variant: the better of no split and the largest
// allowed split by the prediction above.
// SGEMM_SPLITK = S forces min(S, the largest allowed) for sweeps.
int lowp_splits(int variant, int M, int N, int K, long batch = 1, bool ops = false) {
    const int s = lowp_max_splits(variant, M, N, K, batch, ops);
    if (knobs().splitk > 0) return std::min(s, knobs().splitk);
    return s > 1 && lowp_predict_us(variant, s, M, N, K, batch) < lowp_predict_us(variant, 1, M, N, K, batch) ? s
                                                                                                              : 1;
}

// Automatic choice among the 128x128 two-stage kernel (up to two workgroups
// per compute unit, split-K), the 256x128 three-stage kernel and the
// 256x256 and 128x128 four-stage kernels with the alternating schedule (one
// workgroup per compute unit): the least predicted time.  Shapes none of
// them takes run the plain kernel.
// (transposed operands: the two alternating kernels, which are the ones
// built for them)
int lowp_auto(int M, int N, int K, const void *A, int lda, const void *B, int ldb, bool ta = false,
              bool tb = false, long batch = 1) {
    int best = 0;
    double best_t = 0.0;
    for (int id : {1, 2, 4, 5}) {
        if ((ta || tb) && !lowp_takes_ops(id)) continue;
        if (!lowp_fast_ok(kLowpVariants[id], M, N, K, A, lda, B, ldb, ta, tb)) continue;
        const int s = lowp_splits(id, M, N, K, batch, ta || tb);
        const double t = lowp_predict_us(id, s, M, N, K, batch);
        if (best == 0 || t < best_t) {
            best = id;
            best_t = t;
        }
    }
    return best;
}

// 16-bit operands the direct-to-LDS kernels cannot take (rows not 16-byte
// aligned, or K or N not a multiple of 8) otherwise run on the plain kernel
// at 58-65 TFLOP/s against 1000-1300 for the fast kernels (3000x5000x2047,
// 4096^3 with odd leading dimensions).  A large enough problem (or each
// problem of a strided batch) instead copies
// op(A) into an M x K8 and op(B) into a K8 x N8 row-major buffer (stored
// transposed operands are transposed on the way; K8, N8: K and N rounded up
// to multiples of 8; padding zero, so the sums are unchanged; B's padding
// columns only reach accumulators that are never stored) and runs the fast
// kernels on the copies with K8 and the true N.

// dst (rows_out x cols_out 16-bit values, leading dimension cols_out, a
// multiple of 8) = src (rows x cols, leading dimension ld_src) padded with
// zeros; one 16-byte chunk of dst per thread per step of a grid-stride loop.
__global__ void __launch_bounds__(256) pack16_kernel(const unsigned short *__restrict__ src, long ld_src, int rows,
                                                     int cols, unsigned short *__restrict__ dst, int rows_out,
                                                     int cols_out, long src_stride, long dst_stride) {
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    src += blockIdx.y * src_stride;      // problem blockIdx.y of a batch
    dst += blockIdx.y * dst_stride;
    const long q8 = cols_out / 8;
    const long n = (long)rows_out * q8;
    for (long q = blockIdx.x * 256L + threadIdx.x; q < n; q += (long)gridDim.x * 256) {
        const long r = q / q8;
        const int c = (int)(q - r * q8) * 8;
        u16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (r < rows && c + e < cols) ? src[r * ld_src + c + e] : (unsigned short)0;
        *reinterpret_cast<u16x8 *>(dst + r * (long)cols_out + c) = v;
    }
}

// dst[r][c] (rows_out x cols_out 16-bit values, leading dimension cols_out)
// = src[c][r] (src: cols x rows, leading dimension ld_src) for r < rows and
// c < cols, else zero: 32x32 tiles through LDS, both sides coalesced.
__global__ void __launch_bounds__(256) transpose16_kernel(const unsigned short *__restrict__ src, long ld_src,
                                                          int rows, int cols, unsigned short *__restrict__ dst,
                                                          int rows_out, int cols_out, long src_stride,
                                                          long dst_stride) {
    __shared__ unsigned short t[32][33];
    const int r0 = blockIdx.y * 32, c0 = blockIdx.x * 32;
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    src += blockIdx.z * src_stride;      // problem blockIdx.z of a batch
    dst += blockIdx.z * dst_stride;
#pragma unroll
    for (int i = ty; i < 32; i += 8) {
        const int c = c0 + i, r = r0 + tx;           // source row c, column r
        t[i][tx] = (c < cols && r < rows) ? src[(long)c * ld_src + r] : (unsigned short)0;
    }
    __syncthreads();
#pragma unroll
    for (int i = ty; i < 32; i += 8) {
        const int r = r0 + i, c = c0 + tx;
        if (r < rows_out && c < cols_out) dst[(long)r * cols_out + c] = t[tx][i];
    }
}

hipError_t launch_pack16(const void *src, long ld_src, int rows, int cols, void *dst, int rows_out, int cols_out,
                         hipStream_t s, int batch = 1, long src_stride = 0, long dst_stride = 0) {
    const long n = (long)rows_out * (cols_out / 8);
    const long blocks = std::min(ceil_div(n, 256), std::max(4096L / batch, 16L));
    return launch_k(pack16_kernel, dim3((unsigned)blocks, (unsigned)batch), dim3(256), s,
                    static_cast<const unsigned short *>(src), ld_src, rows, cols, static_cast<unsigned short *>(dst),
                    rows_out, cols_out, src_stride, dst_stride);
}

// Whether a 16-bit problem or strided batch that no fast kernel takes
// (operands transposed or not; copies_a / copies_b distinct operands copied)
// is copied: K of at least one K tile, not under graph capture, copies
// within 4 GiB, and the copies' traffic (at about 3 TB/s) plus about 6 us
// for the two extra launches taking less time than the plain kernel's
// product (at 60 TFLOP/s).  SGEMM_PACK = 1 / -1 forces it on / off (where it can run).
bool lowp_copy_plan(int M, int N, int K, void *stream, int batch = 1, int copies_a = 1, int copies_b = 1) {
    if (knobs().pack < 0 || K < 64) return false;
    if (capturing(reinterpret_cast<hipStream_t>(stream))) return false;
    const long K8 = (K + 7) & ~7L, N8 = (N + 7) & ~7L;
    if (ceil_div(M, 32) > 65535 || ceil_div(K8, 32) > 65535) return false;   // transpose grids
    const double copied = 2.0 * ((double)copies_a * M * K8 + (double)copies_b * K8 * N8);
    if (copied > kCopyMaxBytes) return false;
    // (the copies' rows fit the smallest fast tile's 31-bit buffer ranges)
    if (!lowp_fast_ok(kLowpVariants[1], M, (int)N8, (int)K8, nullptr, (int)K8, nullptr, (int)N8)) return false;
    if (knobs().pack > 0) return true;
    return 2.0 * copied / 3e12 + 6e-6 < 2.0 * batch * M * (double)N * K / 60e12;
}

int run_lowp(int dtype, int op_a, int op_b, int M, int N, int K, float alpha, const void *A, int lda,
             const void *B, int ldb, float beta, float *C, int ldc, void *stream, int variant,
             long long sA, long long sB, long long sC, int batch, bool padded_b);

// Whether the fast kernels on the copies can take an untransposed operand
// as it is instead of a copy of it: 16-byte aligned rows whose length
// (`cols`, K for A and N for B) and K are multiples of 8, so that the
// padded K8 and N8 are K and N; in a batch, a stride of whole chunks.
bool lowp_keeps(const void *X, int ldx, int cols, int K, long long stride, int batch) {
    return aligned16(X) && ldx % 8 == 0 && cols % 8 == 0 && K % 8 == 0 && (batch <= 1 || stride % 8 == 0);
}

// The 16-bit product on zero-padded row-major copies of op(A) and op(B)
// (transposed operands transposed on the way); an untransposed operand the
// fast kernels take as it is (lowp_keeps) is used in place.  In a batch, an
// operand of stride 0 is copied once and each other one per problem
// (strides of the copies: multiples of 128 elements).  Returns kUnavailable,
// with nothing enqueued, when the stream's copy buffer is held by another
// call.
int run_lowp_copied(int dtype, bool ta, bool tb, int M, int N, int K, float alpha, const void *A, int lda,
                    long long sA, const void *B, int ldb, long long sB, float beta, float *C, int ldc,
                    long long sC, int batch, void *stream) {
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int K8 = (K + 7) & ~7, N8 = (N + 7) & ~7;
    const int na = batch > 1 && sA != 0 ? batch : 1, nb = batch > 1 && sB != 0 ? batch : 1;
    const size_t a_one = ((size_t)M * K8 + 127) & ~(size_t)127, b_one = ((size_t)K8 * N8 + 127) & ~(size_t)127;
    bool ca = ta || !lowp_keeps(A, lda, K, K, sA, batch);
    bool cb = tb || !lowp_keeps(B, ldb, N, K, sB, batch);
    // the fast kernels on the copies: chosen for the padded width, run on the
    // true one (their loads of B's last chunk read the zero padding); the
    // copies are 16-byte aligned (null stands for them here)
    auto pick = [&] {
        return lowp_auto(M, N8, K8, ca ? nullptr : A, ca ? K8 : lda, cb ? nullptr : B, cb ? N8 : ldb, false, false,
                         batch);
    };
    int v = pick();
    if (v == 0 && !(ca && cb)) {      // an operand in place is outside the kernels' ranges: copy both
        ca = cb = true;
        v = pick();
    }
    if (v == 0) return SGEMM_STATUS_UNSUPPORTED;
    const size_t a_elems = ca ? a_one * na : 0, b_elems = cb ? b_one * nb : 0;
    Lease lease;
    const int st = acquire_slot(kCopySlot, s, (a_elems + b_elems) * 2, lease);
    if (st != SGEMM_STATUS_OK) return st;
    unsigned short *Ap = static_cast<unsigned short *>(lease.mem), *Bp = Ap + a_elems;
    const long src_a = na > 1 ? (long)sA : 0, src_b = nb > 1 ? (long)sB : 0;
    hipError_t e = hipSuccess;
    if (ca)
        e = ta   // stored K x M
                ? launch_k(transpose16_kernel,
                           dim3((unsigned)ceil_div(K8, 32), (unsigned)ceil_div(M, 32), (unsigned)na), dim3(256), s,
                           static_cast<const unsigned short *>(A), (long)lda, M, K, Ap, M, K8, src_a, (long)a_one)
                : launch_pack16(A, lda, M, K, Ap, M, K8, s, na, src_a, (long)a_one);
    if (e == hipSuccess && cb)
        e = tb   // stored N x K
                ? launch_k(transpose16_kernel, dim3((unsigned)ceil_div(N8, 32), (unsigned)ceil_div(K8, 32), (unsigned)nb),
                           dim3(256), s, static_cast<const unsigned short *>(B), (long)ldb, K, N, Bp, K8, N8, src_b,
                           (long)b_one)
                : launch_pack16(B, ldb, K, N, Bp, K8, N8, s, nb, src_b, (long)b_one);
    if (e != hipSuccess) return finish(e, lease, s);
    const long long pa = ca ? (na > 1 ? (long long)a_one : 0) : (batch > 1 ? sA : 0);
    const long long pb = cb ? (nb > 1 ? (long long)b_one : 0) : (batch > 1 ? sB : 0);
    const int prod = run_lowp(dtype, SGEMM_OP_N, SGEMM_OP_N, M, N, K8, alpha, ca ? (const void *)Ap : A,
                              ca ? K8 : lda, cb ? (const void *)Bp : B, cb ? N8 : ldb, beta, C, ldc, stream, v, pa, pb,
                              sC, batch, true);
    const int rel = release_slot(lease, s);
    return prod != SGEMM_STATUS_OK ? prod : rel;
}

int run_lowp(int dtype, int op_a, int op_b, int M, int N, int K, float alpha, const void *A, int lda,
             const void *B, int ldb, float beta, float *C, int ldc, void *stream, int variant,
             long long sA = 0, long long sB = 0, long long sC = 0, int batch = 1, bool padded_b = false) {
    if (dtype != SGEMM_DTYPE_BF16 && dtype != SGEMM_DTYPE_F16) return SGEMM_STATUS_INVALID_DTYPE;
    if ((op_a != SGEMM_OP_N && op_a != SGEMM_OP_T) || (op_b != SGEMM_OP_N && op_b != SGEMM_OP_T))
        return SGEMM_STATUS_INVALID_OP;
    const bool ta = op_a == SGEMM_OP_T, tb = op_b == SGEMM_OP_T;
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_DIM;
    const int need_lda = ta ? (M > 1 ? M : 1) : (K > 1 ? K : 1);
    const int need_ldb = tb ? (K > 1 ? K : 1) : (N > 1 ? N : 1);
    if (lda < need_lda || ldb < need_ldb || ldc < (N > 1 ? N : 1)) return SGEMM_STATUS_INVALID_DIM;
    if (batch < 0 || batch > kMaxBatch) return SGEMM_STATUS_INVALID_DIM;
    if (batch > 1 && (sA < 0 || sB < 0 || (M > 0 && N > 0 && sC < (long long)(M - 1) * ldc + N)))
        return SGEMM_STATUS_INVALID_DIM;
    // (padded_b: A and B are the library's zero-padded copies, whose
    // untransposed B may have N not a multiple of 8 but whole chunks)
    if (variant < SGEMM_VARIANT_AUTO || variant >= kNumLowpVariants) return SGEMM_STATUS_INVALID_VARIANT;
    if (M == 0 || N == 0 || batch == 0) return SGEMM_STATUS_OK;
    if (C == nullptr || (K > 0 && (A == nullptr || B == nullptr))) return SGEMM_STATUS_NULL_POINTER;
    const float *Af = static_cast<const float *>(A), *Bf = static_cast<const float *>(B);
    if (ceil_div(M, 64) * ceil_div(N, 64) > 0x7fffffffL) return SGEMM_STATUS_INVALID_DIM;
    // the fast kernels' 16-byte loads need every problem of a batch aligned
    // like the first: strides of A and B that are multiples of 8 elements
    const bool strides8 = batch <= 1 || (sA % 8 == 0 && sB % 8 == 0);
    if (variant == SGEMM_VARIANT_AUTO) {
        variant = strides8 ? lowp_auto(M, N, K, A, lda, B, ldb, ta, tb, batch) : 0;
        const int na = batch > 1 && sA != 0 ? batch : 1, nb = batch > 1 && sB != 0 ? batch : 1;
        if (variant == 0 && lowp_copy_plan(M, N, K, stream, batch, na, nb)) {
            const int st = run_lowp_copied(dtype, ta, tb, M, N, K, alpha, A, lda, sA, B, ldb, sB, beta, C, ldc, sC,
                                           batch, stream);
            if (st != kUnavailable) return st;
        }
    }
    const LowpVariant &v = kLowpVariants[variant];
    if (variant > 0 && (((ta || tb) && !lowp_takes_ops(variant)) || !strides8)) return SGEMM_STATUS_UNSUPPORTED;
    if (variant > 0 && !lowp_fast_ok(v, M, padded_b ? (N + 7) & ~7 : N, K, A, lda, B, ldb, ta, tb))
        return SGEMM_STATUS_UNSUPPORTED;
    Args a;
    a.A = Af;
    a.B = Bf;
    a.C = C;
    a.lda = lda;
    a.ldb = ldb;
    a.ldc = ldc;
    a.M = M;
    a.N = N;
    a.K = K;
    a.alpha = alpha;
    a.beta = beta;
    a.tiles_m = a.tiles_n = 0;   // set by each launcher from its tile
    a.group_m = knobs().group_m;
    a.xcd_remap = knobs().xcd_remap;
    a.splits = 1;
    a.tile_base = a.tile_count = 0;
    a.ws = nullptr;
    a.counters = nullptr;
    a.strideA = batch > 1 ? (long)sA : 0;
    a.strideB = batch > 1 ? (long)sB : 0;
    a.strideC = batch > 1 ? (long)sC : 0;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    Lease lease;
    const int ws = attach_workspace(a, lowp_splits(variant, M, N, K, batch, ta || tb), s, lease);
    if (ws != SGEMM_STATUS_OK) return ws;
    const bool f16 = dtype == SGEMM_DTYPE_F16;
    return finish(variant > 0 ? launch_lowp_tile(a, f16, variant - 1, ta, tb, batch, s)
                              : launch_simple_lowp(a, f16, ta, tb, batch, s),
                  lease, s);
}

}  // namespace

extern "C" {

int sgemm_lowp(int dtype, int M, int N, int K, float alpha, const void *A, int lda, const void *B, int ldb,
               float beta, float *C, int ldc, void *stream) {
    return run_lowp(dtype, SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream,
                    SGEMM_VARIANT_AUTO);
}

int sgemm_lowp_ex(int dtype, int M, int N, int K, float alpha, const void *A, int lda, const void *B, int ldb,
                  float beta, float *C, int ldc, void *stream, int variant) {
    return run_lowp(dtype, SGEMM_OP_N, SGEMM_OP_N, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

int sgemm_lowp_op(int dtype, int op_a, int op_b, int M, int N, int K, float alpha, const void *A, int lda,
                  const void *B, int ldb, float beta, float *C, int ldc, void *stream, int variant) {
    return run_lowp(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

int sgemm_lowp_strided_batched(int dtype, int op_a, int op_b, int M, int N, int K, float alpha, const void *A,
                               int lda, long long stride_a, const void *B, int ldb, long long stride_b, float beta,
                               float *C, int ldc, long long stride_c, int batch, void *stream) {
    return run_lowp(dtype, op_a, op_b, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, SGEMM_VARIANT_AUTO,
                    stride_a, stride_b, stride_c, batch);
}

int sgemm_lowp_select_variant(int M, int N, int K, const void *A, int lda, const void *B, int ldb) {
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_DIM;
    return lowp_auto(M, N, K, A, lda, B, ldb);
}

int sgemm_lowp_split_factor(int variant, int M, int N, int K) {
    if (variant < 0 || variant >= kNumLowpVariants) return SGEMM_STATUS_INVALID_VARIANT;
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_DIM;
    return lowp_splits(variant, M, N, K);
}

const char *sgemm_lowp_variant_name(int variant) {
    return variant >= 0 && variant < kNumLowpVariants ? kLowpVariants[variant].name : nullptr;
}


int sgemm(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
          float beta, float *C, int ldc, void *stream) {
    return run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, SGEMM_VARIANT_AUTO);
}

int sgemm_noalloc(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
                  float beta, float *C, int ldc, void *stream) {
    return run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, SGEMM_VARIANT_AUTO, true);
}

int sgemm_ex(int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream, int variant) {
    return run(M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream, variant);
}

int sgemm_select_variant(int M, int N, int K, const float *A, int lda, const float *B, int ldb,
                         float beta, const float *C, int ldc) {
    const int st = check_args(M, N, K, A, lda, B, ldb, C, ldc);
    if (st != SGEMM_STATUS_OK) return st;
    return auto_variant(M, N, K, A, lda, B, ldb, beta, C, ldc);
}

int sgemm_num_variants(void) { return kNumVariants; }

const char *sgemm_variant_name(int variant) {
    if (variant < 0 || variant >= kNumVariants) return nullptr;
    return kVariants[variant].name;
}

int sgemm_variant_info(int variant, int *bm, int *bn, int *bk, int *needs_vec) {
    if (variant < 0 || variant >= kNumVariants) return SGEMM_STATUS_INVALID_VARIANT;
    const VariantDesc &d = kVariants[variant];
    if (bm) *bm = d.bm;
    if (bn) *bn = d.bn;
    if (bk) *bk = d.bk;
    if (needs_vec) *needs_vec = d.needs_vec ? 1 : 0;
    return SGEMM_STATUS_OK;
}

int sgemm_op(int op_a, int op_b, int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream) {
    return run_general(op_a, op_b, M, N, K, alpha, A, lda, 0, B, ldb, 0, beta, C, ldc, 0, 1, stream);
}

int sgemm_strided_batched(int op_a, int op_b, int M, int N, int K, float alpha, const float *A, int lda,
                          long long stride_a, const float *B, int ldb, long long stride_b, float beta, float *C,
                          int ldc, long long stride_c, int batch, void *stream) {
    return run_general(op_a, op_b, M, N, K, alpha, A, lda, stride_a, B, ldb, stride_b, beta, C, ldc, stride_c, batch,
                       stream);
}

// Column-major (BLAS) calls: a column-major matrix is the row-major storage
// of its transpose, so C = op(A) op(B) in column-major storage is the
// row-major product C^T = op(B)^T op(A)^T: the operands trade places, and so
// do M and N and the two ops.
int sgemm_cm(int op_a, int op_b, int M, int N, int K, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream) {
    return run_general(op_b, op_a, N, M, K, alpha, B, ldb, 0, A, lda, 0, beta, C, ldc, 0, 1, stream);
}

int sgemm_cm_strided_batched(int op_a, int op_b, int M, int N, int K, float alpha, const float *A, int lda,
                             long long stride_a, const float *B, int ldb, long long stride_b, float beta, float *C,
                             int ldc, long long stride_c, int batch, void *stream) {
    return run_general(op_b, op_a, N, M, K, alpha, B, ldb, stride_b, A, lda, stride_a, beta, C, ldc, stride_c, batch,
                       stream);
}

int sgemm_split_factor(int variant, int M, int N, int K) {
    if (variant < 0 || variant >= kNumVariants) return SGEMM_STATUS_INVALID_VARIANT;
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_DIM;
    const VariantDesc &d = kVariants[variant];
    if (!d.split_k || M == 0 || N == 0) return 1;
    return choose_splits(M, N, K, d.bm, d.bn, d.bk);
}

int sgemm_tail_split(int variant, int M, int N, int K, int *tail_tiles) {
    if (tail_tiles) *tail_tiles = 0;
    if (variant < 0 || variant >= kNumVariants) return SGEMM_STATUS_INVALID_VARIANT;
    if (M < 0 || N < 0 || K < 0) return SGEMM_STATUS_INVALID_DIM;
    const VariantDesc &d = kVariants[variant];
    if (!d.split_k || M == 0 || N == 0 || choose_splits(M, N, K, d.bm, d.bn, d.bk) > 1) return 1;
    // the lean kernel's operand checks with packed leading dimensions
    Args a{};
    a.M = M;
    a.N = N;
    a.K = K;
    a.lda = K > 1 ? K : 1;
    a.ldb = N > 1 ? N : 1;
    const int s = choose_tail_splits(d, a);
    if (s > 1 && tail_tiles) *tail_tiles = (int)((ceil_div(M, d.bm) * ceil_div(N, d.bn)) % kTailSlots);
    return s;
}

const char *sgemm_strerror(int status) {
    switch (status) {
        case SGEMM_STATUS_OK: return "ok";
        case SGEMM_STATUS_INVALID_DIM: return "invalid dimension or leading dimension";
        case SGEMM_STATUS_NULL_POINTER: return "NULL pointer with a non-empty extent";
        case SGEMM_STATUS_HIP_ERROR: return "HIP runtime error";
        case SGEMM_STATUS_INVALID_VARIANT: return "unknown kernel variant";
        case SGEMM_STATUS_UNSUPPORTED: return "variant needs 16-byte aligned pointers and leading dimensions";
        case SGEMM_STATUS_INVALID_OP: return "operation code is neither SGEMM_OP_N nor SGEMM_OP_T";
        case SGEMM_STATUS_INVALID_DTYPE: return "input type is neither SGEMM_DTYPE_BF16 nor SGEMM_DTYPE_F16";
        case SGEMM_STATUS_SCRATCH_TOO_SMALL:
            return "sgemm_noalloc: the split of K needs more scratch than SGEMM_NOALLOC_SCRATCH_BYTES";
        default: return "unknown status";
    }
}

const char *sgemm_last_hip_error(void) { return g_last_hip_error; }

int sgemm_version(void) { return SGEMM_LIB_VERSION; }

long long sgemm_workspace_bytes(void) {
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record_hip_error(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(g_slot_mu);
    long long total = 0;
    for (const Slot &x : g_slots)
        if (x.dev == dev) total += (long long)x.bytes;
    return total;
}

int sgemm_release_workspaces(void) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return record_hip_error(e, "hipGetDevice");
    std::vector<std::list<Slot>::iterator> victims;
    {
        std::lock_guard<std::mutex> lock(g_slot_mu);
        for (auto it = g_slots.begin(); it != g_slots.end(); ++it) {
            if (it->dev != dev || it->users > 0 || it->moving || it->pinned) continue;
            it->moving = true;
            victims.push_back(it);
        }
    }
    int st = SGEMM_STATUS_OK;
    std::vector<std::list<Slot>::iterator> freed;
    // a last use that no event marks: wait for the whole device, once
    hipError_t drain = hipSuccess;
    for (auto it : victims) {
        if (it->last_use == kUnmarked) {
            drain = hipDeviceSynchronize();
            break;
        }
    }
    for (auto it : victims) {
        // the slot's last use must be over before its memory goes
        if (it->last_use == kUnmarked) {
            e = drain;
        } else {
            e = it->last_use == kEventMarks ? hipEventSynchronize(it->done) : hipSuccess;
        }
        if (e == hipSuccess && it->mem != nullptr) e = hipFree(it->mem);
        if (e != hipSuccess) {
            if (st == SGEMM_STATUS_OK) st = record_hip_error(e, "releasing a buffer");
            std::lock_guard<std::mutex> lock(g_slot_mu);
            it->moving = false;
            it->pinned = true;      // state unknown: never reused
            continue;
        }
        if (it->done != nullptr) (void)hipEventDestroy(it->done);
        freed.push_back(it);
    }
    std::lock_guard<std::mutex> lock(g_slot_mu);
    for (auto it : freed) g_slots.erase(it);
    return st;
}

}  // extern "C"

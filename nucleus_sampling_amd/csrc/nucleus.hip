// nucleus.hip -- the C ABI of libnucleus (declared in include/nucleus.h):
// argument validation, launch-shape choice and launches on the caller's
// stream.  No call synchronises the device or allocates memory.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>
#include <chrono>
#include <mutex>

#include "nucleus.h"
#include "common.h"
#include "params.h"
#include "rejection.h"
#include "rowpath.h"
#include "sampler.h"
#include "spec.h"
#include "stream_read.h"
#include "workspace.h"

using namespace nucleus;

namespace {

// The library is built for gfx950 only; refuse other devices up front rather
// than fail inside a launch.
int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NUCLEUS_EDEVICE;
    static std::mutex mu;
    static int known[64] = {0};  // 0 unknown, 1 ok, -1 unsupported
    if (dev < 0 || dev >= 64) return NUCLEUS_EDEVICE;
    std::lock_guard<std::mutex> lock(mu);
    if (known[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return NUCLEUS_EDEVICE;
        known[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    }
    return known[dev] == 1 ? NUCLEUS_OK : NUCLEUS_EDEVICE;
}

// By default a row runs on one workgroup of its own (row_kernel, every
// phase).  Small batches of long rows split each row over ceil(V / kChunk)
// register-resident workgroups instead (tile_kernel): fewer than 128 rows of
// more than 32768 tokens, and at most 1536 workgroups in all.  Measured on
// MI355X (Normal logits, T = 1): with rows of 8192 or 32000 tokens one
// workgroup per row is as fast or faster at every batch size; with 128256
// tokens splitting wins up to ~64-96 rows (45 against 67 us at B = 1, 62
// against 80 us at B = 64) and loses at 127 (108 against 84 us).  The
// chunked-race path (row_kernel's histogram passes, then race_kernel spread
// over the device) is taken on request.
constexpr int64_t kSplitBelowRows = 128;
constexpr int64_t kSplitAboveTokens = 32768;
constexpr int64_t kSplitMaxWorkgroups = 1536;

enum Path { kPathTile, kPathRows, kPathFused };

// Workgroups per row of the split-row path, 0 if rows are too long for it.
int tile_chunks(int64_t V)
{
    const int64_t K = (V + kChunk - 1) / kChunk;
    return K <= kMaxChunks ? (int)K : 0;
}

// The path a call takes; -1 for a flag combination that cannot run.
int choose_path(int64_t B, int64_t V, int32_t flags)
{
    const int32_t known = NUCLEUS_FLAG_SINGLE_WORKGROUP | NUCLEUS_FLAG_SPLIT_ROWS | NUCLEUS_FLAG_ROW_RACE;
    if ((flags & ~known) || __builtin_popcount((unsigned)flags) > 1) return -1;
    if (flags & NUCLEUS_FLAG_SINGLE_WORKGROUP) return kPathFused;
    if (flags & NUCLEUS_FLAG_ROW_RACE) return kPathRows;
    if (flags & NUCLEUS_FLAG_SPLIT_ROWS) return tile_chunks(V) ? kPathTile : -1;
    const int64_t K = tile_chunks(V);
    return (B < kSplitBelowRows && V > kSplitAboveTokens && K && B * K <= kSplitMaxWorkgroups) ? kPathTile
                                                                                               : kPathFused;
}

size_t path_workspace(int path, int64_t B, int64_t V)
{
    if (B == 0) return 0;
    if (path == kPathTile) return work_layout(B, tile_chunks(V), kBins).total;
    if (path == kPathRows) return row_work_bytes(B, nullptr);
    return 0;
}

// A distinct 56-bit tag per call.  The sequence starts at a value derived
// from this process (so tags of different processes rarely meet) and steps
// by one; stale barrier words never carry the current tag.
uint64_t next_epoch()
{
    static std::atomic<uint64_t> counter{0};
    static const uint64_t base = [] {
        const uint64_t t = (uint64_t)std::chrono::high_resolution_clock::now().time_since_epoch().count();
        return (t * 0x9E3779B97F4A7C15ull) ^ ((uint64_t)(uintptr_t)&counter << 17);
    }();
    return (base + counter.fetch_add(1) + 1) & ((uint64_t(1) << 56) - 1);
}

// Workgroups of race_kernel that fit on the current device at once (its
// occupancy times the CU count), per dtype; 0 if the runtime cannot say.
int64_t race_workgroups(int32_t dtype)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    static std::mutex mu;
    static int64_t known[64][2] = {};
    std::lock_guard<std::mutex> lock(mu);
    int64_t& k = known[dev][dtype == NUCLEUS_BF16 ? 1 : 0];
    if (k == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        const hipError_t e = dtype == NUCLEUS_BF16
                                 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, race_kernel<kBF16>, kRaceThreads, 0)
                                 : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, race_kernel<kF32>, kRaceThreads, 0);
        if (e != hipSuccess || per_cu < 1) return 0;
        k = (int64_t)cus * per_cu;
    }
    return k;
}

template <class T>
bool aligned(const T* p)
{
    return ((uintptr_t)p % alignof(T)) == 0;
}

// Whether a call asks for the pre-chain (penalties or a grammar mask).
bool has_prechain(const nucleus_options* opt)
{
    return opt && (opt->allowed_mask || opt->history_len != 0 || opt->history || opt->repetition_penalty ||
                   opt->frequency_penalty || opt->presence_penalty);
}

// The scratch of nucleus_sample_noalloc: one static array per GPU, never
// allocated by a call.  In host code the array's name stands for a host-side
// shadow, not a device address: every use goes through the address
// hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// The current device's address of `scratch`, looked up once per device;
// nullptr if the runtime cannot give it.
void* static_scratch()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    static std::mutex mu;
    static void* known[64] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (!known[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        known[dev] = ptr;
    }
    return known[dev];
}

// Phase clocks (builds with NUCLEUS_PHASE_STAMPS only): the buffer later
// calls of the one-workgroup-per-row path write to.
std::atomic<uint64_t*> g_stamps{nullptr};
std::atomic<int64_t> g_stamp_rows{0};

uint64_t* stamps_for(int64_t B)
{
#ifdef NUCLEUS_PHASE_STAMPS
    uint64_t* s = g_stamps.load();
    return (s && B <= g_stamp_rows.load()) ? s : nullptr;
#else
    (void)B;
    return nullptr;
#endif
}

}  // namespace

extern "C" {

int nucleus_version(void) { return 260; }

int nucleus_phase_stamps(uint64_t* buf, int64_t rows)
{
#ifdef NUCLEUS_PHASE_STAMPS
    if (rows < 0 || (buf && (uintptr_t)buf % 8)) return NUCLEUS_EINVAL;
    g_stamp_rows.store(buf ? rows : 0);
    g_stamps.store(buf);
    return NUCLEUS_OK;
#else
    (void)buf;
    (void)rows;
    return NUCLEUS_EINVAL;
#endif
}

const char* nucleus_strerror(int code)
{
    switch (code) {
    case NUCLEUS_OK: return "ok";
    case NUCLEUS_EINVAL: return "invalid argument";
    case NUCLEUS_EWORKSPACE: return "workspace missing or too small";
    case NUCLEUS_ELAUNCH: return "kernel launch failed";
    case NUCLEUS_EDEVICE: return "no usable gfx950 device";
    default: return "unknown error";
    }
}

size_t nucleus_workspace_bytes_for(int64_t B, int64_t V, int32_t dtype, int32_t flags)
{
    if (B < 0 || V < 1 || V >= (int64_t(1) << 31) || (dtype != NUCLEUS_F32 && dtype != NUCLEUS_BF16)) return 0;
    const int path = choose_path(B, V, flags);
    return path < 0 ? 0 : path_workspace(path, B, V);
}

size_t nucleus_workspace_bytes(int64_t B, int64_t V, int32_t dtype)
{
    return nucleus_workspace_bytes_for(B, V, dtype, 0);
}

int nucleus_sample(const void* logits, int64_t B, int64_t V, const float* temperature, const float* top_p,
                   const int32_t* top_k, const float* min_p, uint64_t seed, uint64_t step, int32_t* out_token,
                   int32_t* out_keep_count, float* out_probs, const nucleus_options* opt)
{
    const int32_t dtype = opt ? opt->dtype : NUCLEUS_F32;
    const int64_t stride = (opt && opt->row_stride) ? opt->row_stride : V;
    if (B < 0 || V < 1 || V >= (int64_t(1) << 31) || stride < V) return NUCLEUS_EINVAL;
    if (dtype != NUCLEUS_F32 && dtype != NUCLEUS_BF16) return NUCLEUS_EINVAL;
    if (opt && opt->split_give_up_row < 0) return NUCLEUS_EINVAL;
    const bool pre = has_prechain(opt);
    if (pre) {
        if (opt->history_len < 0 || opt->history_len > kHistMax || (opt->history_len > 0 && !opt->history))
            return NUCLEUS_EINVAL;
        if ((V + 31) / 32 > kMaskWordsMax) return NUCLEUS_EINVAL;  // the per-token bits are staged in LDS
        if (opt->flags & (NUCLEUS_FLAG_SPLIT_ROWS | NUCLEUS_FLAG_ROW_RACE)) return NUCLEUS_EINVAL;
        if ((opt->history && !aligned(opt->history)) || (opt->repetition_penalty && !aligned(opt->repetition_penalty)) ||
            (opt->frequency_penalty && !aligned(opt->frequency_penalty)) ||
            (opt->presence_penalty && !aligned(opt->presence_penalty)) ||
            (opt->allowed_mask && !aligned(opt->allowed_mask)))
            return NUCLEUS_EINVAL;
    }
    const int path = pre ? (choose_path(B, V, opt->flags) < 0 ? -1 : kPathFused) : choose_path(B, V, opt ? opt->flags : 0);
    if (path < 0) return NUCLEUS_EINVAL;
    if (B == 0) return NUCLEUS_OK;
    if (!logits || !temperature || !top_p || !out_token || !out_keep_count) return NUCLEUS_EINVAL;
    const size_t esz = dtype == NUCLEUS_F32 ? 4 : 2;
    if ((uintptr_t)logits % esz != 0 || !aligned(temperature) || !aligned(top_p) || (top_k && !aligned(top_k)) ||
        (min_p && !aligned(min_p)) || !aligned(out_token) || !aligned(out_keep_count) ||
        (out_probs && !aligned(out_probs)) || (opt && opt->out_min_kept_logit && !aligned(opt->out_min_kept_logit)) ||
        (opt && opt->seeds && !aligned(opt->seeds)) || (opt && opt->out_logprobs && !aligned(opt->out_logprobs)))
        return NUCLEUS_EINVAL;
    const size_t need = path_workspace(path, B, V);
    if (need > 0 && (!opt || !opt->workspace || opt->workspace_bytes < need || (uintptr_t)opt->workspace % 256))
        return NUCLEUS_EWORKSPACE;
    const int dev_rc = check_device();
    if (dev_rc != NUCLEUS_OK) return dev_rc;

    Params p;
    p.logits = logits;
    p.B = B;
    p.V = V;
    p.stride = stride;
    p.temperature = temperature;
    p.top_p = top_p;
    p.top_k = top_k;
    p.min_p = min_p;
    p.seed_lo = (uint32_t)seed;
    p.seed_hi = (uint32_t)(seed >> 32);
    p.step_lo = (uint32_t)step;
    p.step_hi = (uint32_t)(step >> 32);
    p.out_token = out_token;
    p.out_count = out_keep_count;
    p.out_probs = out_probs;
    p.out_min_kept = opt ? opt->out_min_kept_logit : nullptr;
    p.seeds = opt ? opt->seeds : nullptr;
    p.out_logprobs = opt ? opt->out_logprobs : nullptr;
    p.hist = pre ? opt->history : nullptr;
    p.hist_len = pre ? opt->history_len : 0;
    p.rep_pen = pre ? opt->repetition_penalty : nullptr;
    p.freq_pen = pre ? opt->frequency_penalty : nullptr;
    p.pres_pen = pre ? opt->presence_penalty : nullptr;
    p.allowed = pre ? opt->allowed_mask : nullptr;
    p.stamps = stamps_for(B);
    const size_t vec_bytes = dtype == NUCLEUS_F32 ? 16 : 8;
    p.vec_in = ((uintptr_t)logits % vec_bytes == 0) && ((size_t)stride * esz) % vec_bytes == 0;

    hipStream_t s = opt ? (hipStream_t)opt->stream : nullptr;
    if (path == kPathTile) {
        const int K = tile_chunks(V);
        const WorkLayout L = work_layout(B, K, kBins);
        char* ws = (char*)opt->workspace;
        Work wk;
        wk.ctl = (RowCtl*)(ws + L.ctl);
        wk.slot_a = (uint4*)(ws + L.slot_a);
        wk.slot_h = (uint64_t*)(ws + L.slot_h);
        wk.slot_c = (uint32_t*)(ws + L.slot_c);
        wk.slot_r = (RacePart*)(ws + L.slot_r);
        wk.cand = (uint2*)(ws + L.cand);
        wk.K = K;
        wk.epoch = next_epoch();
        wk.give_up_row = opt->split_give_up_row - 1;  // opt is set: this path needs its workspace
        const dim3 grid((unsigned)(padded_rows(B) * K)), block(kThreads);
        if (dtype == NUCLEUS_F32)
            hipLaunchKernelGGL(tile_kernel<kF32>, grid, block, 0, s, p, wk);
        else
            hipLaunchKernelGGL(tile_kernel<kBF16>, grid, block, 0, s, p, wk);
    } else if (path == kPathRows) {
        size_t cand_off = 0;
        row_work_bytes(B, &cand_off);
        RowWork rw;
        rw.st = (RowPathState*)opt->workspace;
        rw.cand = (uint2*)((char*)opt->workspace + cand_off);
        rw.N = (int)((V + kItemTokens - 1) / kItemTokens);  // race items per row
        const int64_t waves = B * rw.N;
        const int64_t resident = race_workgroups(dtype);
        if (resident <= 0) return NUCLEUS_ELAUNCH;
        const int64_t wgs_needed = (waves + kRaceThreads / kWave - 1) / (kRaceThreads / kWave);
        const int NC = (int)((V + kRaceChunk - 1) / kRaceChunk);  // probability chunks per row
        const dim3 rows((unsigned)B), chunks((unsigned)(padded_rows(B) * NC));
        const dim3 racers((unsigned)(wgs_needed < resident ? wgs_needed : resident));
        RowWork pw = rw;
        pw.N = NC;
        if (dtype == NUCLEUS_F32) {
            hipLaunchKernelGGL((row_kernel<kF32, true>), rows, dim3(kRowThreads), 0, s, p, rw);
            hipLaunchKernelGGL(race_kernel<kF32>, racers, dim3(kRaceThreads), 0, s, p, rw);
            hipLaunchKernelGGL(resolve_kernel<kF32>, rows, dim3(kRowThreads), 0, s, p, rw);
            if (out_probs || p.out_logprobs) hipLaunchKernelGGL(probs_kernel<kF32>, chunks, dim3(kRaceThreads), 0, s, p, pw);
        } else {
            hipLaunchKernelGGL((row_kernel<kBF16, true>), rows, dim3(kRowThreads), 0, s, p, rw);
            hipLaunchKernelGGL(race_kernel<kBF16>, racers, dim3(kRaceThreads), 0, s, p, rw);
            hipLaunchKernelGGL(resolve_kernel<kBF16>, rows, dim3(kRowThreads), 0, s, p, rw);
            if (out_probs || p.out_logprobs) hipLaunchKernelGGL(probs_kernel<kBF16>, chunks, dim3(kRaceThreads), 0, s, p, pw);
        }
    } else {
        const RowWork none = {};
        if (pre && dtype == NUCLEUS_F32)
            hipLaunchKernelGGL((row_kernel<kF32, false, true>), dim3((unsigned)B), dim3(kRowThreads), 0, s, p, none);
        else if (pre)
            hipLaunchKernelGGL((row_kernel<kBF16, false, true>), dim3((unsigned)B), dim3(kRowThreads), 0, s, p, none);
        else if (dtype == NUCLEUS_F32)
            hipLaunchKernelGGL((row_kernel<kF32, false>), dim3((unsigned)B), dim3(kRowThreads), 0, s, p, none);
        else
            hipLaunchKernelGGL((row_kernel<kBF16, false>), dim3((unsigned)B), dim3(kRowThreads), 0, s, p, none);
    }
    return hipGetLastError() == hipSuccess ? NUCLEUS_OK : NUCLEUS_ELAUNCH;
}

int nucleus_sample_noalloc(const void* logits, int64_t B, int64_t V, const float* temperature, const float* top_p,
                           const int32_t* top_k, const float* min_p, uint64_t seed, uint64_t step, int32_t* out_token,
                           int32_t* out_keep_count, float* out_probs, const nucleus_options* opt)
{
    nucleus_options o = {};
    if (opt) o = *opt;
    const int32_t dtype = o.dtype;
    if (B < 0 || V < 1 || V >= (int64_t(1) << 31) || (dtype != NUCLEUS_F32 && dtype != NUCLEUS_BF16))
        return NUCLEUS_EINVAL;
    const int path = has_prechain(&o) ? kPathFused : choose_path(B, V, o.flags);
    if (path < 0) return NUCLEUS_EINVAL;
    if (path_workspace(path, B, V) > kStaticScratchBytes) return NUCLEUS_EWORKSPACE;
    const int dev_rc = check_device();
    if (dev_rc != NUCLEUS_OK) return dev_rc;
    void* ws = static_scratch();
    if (!ws) return NUCLEUS_EDEVICE;
    o.workspace = ws;
    o.workspace_bytes = kStaticScratchBytes;
    return nucleus_sample(logits, B, V, temperature, top_p, top_k, min_p, seed, step, out_token, out_keep_count,
                          out_probs, &o);
}

size_t nucleus_noalloc_scratch_bytes(void) { return kStaticScratchBytes; }

int nucleus_sample_rejection(const void* logits, int64_t B, int64_t V, const float* temperature, const float* top_p,
                             const float* min_p, uint64_t seed, uint64_t step, int32_t* out_token,
                             int32_t* out_rounds, const nucleus_options* opt)
{
    const int32_t dtype = opt ? opt->dtype : NUCLEUS_F32;
    const int64_t stride = (opt && opt->row_stride) ? opt->row_stride : V;
    if (B < 0 || V < 1 || V >= (int64_t(1) << 31) || stride < V) return NUCLEUS_EINVAL;
    if (dtype != NUCLEUS_F32 && dtype != NUCLEUS_BF16) return NUCLEUS_EINVAL;
    if (opt && (opt->flags || opt->out_min_kept_logit || opt->out_logprobs || has_prechain(opt))) return NUCLEUS_EINVAL;
    if (B == 0) return NUCLEUS_OK;
    if (!logits || !temperature || !top_p || !out_token) return NUCLEUS_EINVAL;
    const size_t esz = dtype == NUCLEUS_F32 ? 4 : 2;
    if ((uintptr_t)logits % esz != 0 || !aligned(temperature) || !aligned(top_p) || (min_p && !aligned(min_p)) ||
        !aligned(out_token) || (out_rounds && !aligned(out_rounds)) || (opt && opt->seeds && !aligned(opt->seeds)))
        return NUCLEUS_EINVAL;
    const int dev_rc = check_device();
    if (dev_rc != NUCLEUS_OK) return dev_rc;

    Params p = {};
    p.logits = logits;
    p.B = B;
    p.V = V;
    p.stride = stride;
    p.temperature = temperature;
    p.top_p = top_p;
    p.top_k = nullptr;
    p.min_p = min_p;
    p.seed_lo = (uint32_t)seed;
    p.seed_hi = (uint32_t)(seed >> 32);
    p.step_lo = (uint32_t)step;
    p.step_hi = (uint32_t)(step >> 32);
    p.out_token = out_token;
    p.seeds = opt ? opt->seeds : nullptr;
    const size_t vec_bytes = dtype == NUCLEUS_F32 ? 16 : 8;
    p.vec_in = ((uintptr_t)logits % vec_bytes == 0) && ((size_t)stride * esz) % vec_bytes == 0;
    hipStream_t s = opt ? (hipStream_t)opt->stream : nullptr;
    if (dtype == NUCLEUS_F32)
        hipLaunchKernelGGL(rejection_kernel<kF32>, dim3((unsigned)B), dim3(kRowThreads), 0, s, p, out_rounds);
    else
        hipLaunchKernelGGL(rejection_kernel<kBF16>, dim3((unsigned)B), dim3(kRowThreads), 0, s, p, out_rounds);
    return hipGetLastError() == hipSuccess ? NUCLEUS_OK : NUCLEUS_ELAUNCH;
}

size_t nucleus_spec_workspace_bytes(int64_t B, int64_t V)
{
    if (B < 0 || V < 1 || V >= (int64_t(1) << 31)) return 0;
    return align256((size_t)B * (size_t)((V + kSpecChunk - 1) / kSpecChunk) * 8);
}

int nucleus_spec_verify(const float* target_probs, const float* draft_probs, const int32_t* draft_token, int64_t B,
                        int64_t V, uint64_t seed, uint64_t step, int32_t* out_token, int32_t* out_accepted,
                        const nucleus_options* opt)
{
    if (B < 0 || V < 1 || V >= (int64_t(1) << 31)) return NUCLEUS_EINVAL;
    if (opt && ((opt->row_stride && opt->row_stride != V) || opt->dtype != NUCLEUS_F32 || opt->flags ||
                opt->out_min_kept_logit || opt->out_logprobs || has_prechain(opt)))
        return NUCLEUS_EINVAL;
    if (B == 0) return NUCLEUS_OK;
    if (!target_probs || !draft_probs || !draft_token || !out_token) return NUCLEUS_EINVAL;
    if (!aligned(target_probs) || !aligned(draft_probs) || !aligned(draft_token) || !aligned(out_token) ||
        (out_accepted && !aligned(out_accepted)) || (opt && opt->seeds && !aligned(opt->seeds)))
        return NUCLEUS_EINVAL;
    const size_t need = nucleus_spec_workspace_bytes(B, V);
    if (!opt || !opt->workspace || opt->workspace_bytes < need || (uintptr_t)opt->workspace % 256)
        return NUCLEUS_EWORKSPACE;
    if (B * ((V + kSpecChunk - 1) / kSpecChunk) >= (int64_t(1) << 31)) return NUCLEUS_EINVAL;
    const int dev_rc = check_device();
    if (dev_rc != NUCLEUS_OK) return dev_rc;
    SpecParams sp = {};
    sp.target = target_probs;
    sp.draft = draft_probs;
    sp.draft_token = draft_token;
    sp.B = B;
    sp.V = V;
    sp.seed_lo = (uint32_t)seed;
    sp.seed_hi = (uint32_t)(seed >> 32);
    sp.step_lo = (uint32_t)step;
    sp.step_hi = (uint32_t)(step >> 32);
    sp.seeds = opt ? opt->seeds : nullptr;
    sp.out_token = out_token;
    sp.out_accepted = out_accepted;
    sp.vec = (V % 4 == 0) && (uintptr_t)target_probs % 16 == 0 && (uintptr_t)draft_probs % 16 == 0;
    sp.C = (int)((V + kSpecChunk - 1) / kSpecChunk);
    sp.part = (uint64_t*)opt->workspace;
    hipStream_t s = opt ? (hipStream_t)opt->stream : nullptr;
    hipLaunchKernelGGL(spec_chunk_kernel, dim3((unsigned)(B * sp.C)), dim3(kSpecThreads), 0, s, sp);
    hipLaunchKernelGGL(spec_finish_kernel, dim3((unsigned)((B + 255) / 256)), dim3(256), 0, s, sp);
    return hipGetLastError() == hipSuccess ? NUCLEUS_OK : NUCLEUS_ELAUNCH;
}

int nucleus_stream_read(const void* buf, size_t bytes, uint64_t* sink, void* stream)
{
    if (!buf || !sink || (uintptr_t)buf % 16 != 0 || !aligned(sink)) return NUCLEUS_EINVAL;
    const int dev_rc = check_device();
    if (dev_rc != NUCLEUS_OK) return dev_rc;
    return launch_stream_read(buf, bytes, sink, (hipStream_t)stream) ? NUCLEUS_OK : NUCLEUS_ELAUNCH;
}

}  // extern "C"

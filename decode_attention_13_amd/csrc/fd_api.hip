// fd_api.hip -- the C ABI of include/fd.h: host-side validation, the split
// planner and the kernel launches. Nothing here allocates device memory, and
// every launch goes on the caller's stream; only a paged call with
// fd_options.debug_checks synchronises (it reads back its error record).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cfloat>
#include <climits>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "fd.h"
#include "fd_internal.h"

namespace {

thread_local std::string g_last_error;

fd_status fail(fd_status s, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ilog2_exact(int x) {  // log2 of a power of two, -1 otherwise
    if (x <= 0 || (x & (x - 1)) != 0) return -1;
    int n = 0;
    while ((1 << n) < x) ++n;
    return n;
}

long long pow2_floor(long long x) {
    long long p = 1;
    while (p * 2 <= x) p *= 2;
    return p;
}

// Planner constants (measured on MI355X).
//  - Chunk bounds: long enough to amortise a workgroup's start (q load, first
//    round trip to HBM) and its partial write, short enough to spread short
//    caches over the chip.
// Workgroups aimed at per compute unit (contiguous caches). A split-kernel
// workgroup is 4 waves, each with one or two K/V tiles in flight. Measured over
// 2k-128k tokens: one workgroup per CU is best for MHA with two KV heads packed
// (16-bit and fp32 rows) and for GQA on both kernels (16-bit, fp32 and E4M3
// caches), by up to 15-30% at 8k-32k tokens; two are best for MHA over E4M3
// rows (four KV heads packed, half the bytes per load) and for MHA caches
// under 64 MiB.
int target_wgs_per_cu(fd_dtype dtype, bool mha, long long kv_bytes) {
    if (mha && (fd::is_fp8_cache(dtype) || kv_bytes < (64LL << 20))) return 2;
    return 1;
}
// Paged batches: a workgroup pays a fixed cost (block-table and first KV round
// trips, the end-of-split merge and partial store) worth about kWgFixedBytes of
// streaming at its share of the bandwidth, and a ragged batch ends with about
// half a workgroup of imbalance per resident slot. Balancing the two terms gives
// a workgroup size of sqrt(2 * bytes per slot * kWgFixedBytes). A work-list
// workgroup first loads every sequence length and numbers the items (a prefix
// sum and two barriers) before it can load its table slice: one more dependent
// round trip, and a larger fixed cost. Measured on the GQA4 batch (grid) and
// the GQA8 batch (work list), bf16/f16 caches, with the largest items started
// first: best strides 1024 and 4096 (2048 for the GQA8 batch cost 2.2%).
constexpr double kWgFixedBytes = 32768.0;
// An E4M3 cache halves the bytes of a token but not the per-page and per-split
// work around them (table entries, addresses, the scale, the partial store), so
// its fixed cost is worth twice as many bytes: on the GQA4 batch the split kernel
// ran 117.6 us at 2048 tokens against 125.5 us at 1024, and on the GQA8 batch
// 8192 tokens matched 4096 in the split kernel and saved 2.4% of the step (fewer
// partials to merge).
constexpr double kWgFixedFp8Scale = 2.0;
constexpr double kWgFixedBytesList = 3.0 * kWgFixedBytes;
constexpr int kPagedSlotsPerCu = 2;  // resident split workgroups per CU (two waves per SIMD)
constexpr int kMinChunk = 16;  // one 16-token block: a short cache still spreads over many workgroups
constexpr int kMaxChunk = 16384;
constexpr int kMaxSplits = 4096;
constexpr size_t kErrRecordBytes = 4 * sizeof(int32_t);  // debug record: kind, sequence, index, value

std::mutex g_cu_mutex;
std::vector<int> g_cu_cache;

// Bytes of one cached K or V element.
int cache_elem_bytes(fd_dtype d) {
    if (d == FD_DTYPE_F32) return 4;
    if (fd::is_fp8_cache(d)) return 1;
    return 2;
}

// Heads per workgroup of the vector-ALU kernel: the largest compiled group
// size dividing G (a workgroup reads its KV rows once for all its heads). fp32
// rows stop at 4 heads: 8 heads of fp32 state and rows exceed the registers.
int valu_heads_per_group(int G, fd_dtype dtype) {
    for (int gt : {8, 4, 2, 1})
        if (G % gt == 0 && !(gt == 8 && dtype == FD_DTYPE_F32)) return gt;
    return 1;
}

// The matrix-core kernel takes up to 16 heads (one MFMA tile of columns).
int mfma_heads_per_group(int G) {
    if (G <= 16) return G;
    return G % 16 == 0 ? 16 : 0;
}

// Matrix cores when a group of query heads forms a tile (16-bit inputs, >= 3
// heads per KV head); the vector ALUs otherwise. Measured on one paged batch
// with 2, 3 and 4 query heads per KV head: the vector ALUs lead by 2% at 2, the
// matrix cores by 2.6x at 3 and 3% at 4.
int pick_kernel(fd_dtype dtype, int G, int forced) {
    const bool mfma_ok = fd::query_dtype(dtype) != FD_DTYPE_F32 && mfma_heads_per_group(G) > 0;
    if (forced == FD_KERNEL_VALU) return FD_KERNEL_VALU;
    if (forced == FD_KERNEL_MFMA) return mfma_ok ? FD_KERNEL_MFMA : -1;
    return (mfma_ok && G >= 3) ? FD_KERNEL_MFMA : FD_KERNEL_VALU;
}

fd_status check_common(int B, int H, int Hkv, int D, fd_dtype dtype, const fd_options *opt) {
    if (B < 1 || H < 1 || Hkv < 1) return fail(FD_ERR_INVALID_ARG, "B, H and Hkv must be >= 1 (got %d, %d, %d)", B, H, Hkv);
    if (H % Hkv != 0) return fail(FD_ERR_INVALID_ARG, "H (%d) must be a multiple of Hkv (%d)", H, Hkv);
    if (D != FD_HEAD_DIM) return fail(FD_ERR_UNSUPPORTED, "head dim %d unsupported (only %d)", D, FD_HEAD_DIM);
    if (dtype < FD_DTYPE_F32 || dtype > FD_DTYPE_BF16_KV_E4M3)
        return fail(FD_ERR_UNSUPPORTED, "unknown dtype %d", (int)dtype);
    if (opt) {
        if (opt->force_num_splits < 0 || opt->force_chunk < 0)
            return fail(FD_ERR_INVALID_ARG, "negative force_num_splits/force_chunk");
        if (opt->force_chunk > 0 && opt->force_chunk % FD_CHUNK_QUANTUM != 0)
            return fail(FD_ERR_INVALID_ARG, "force_chunk %d is not a multiple of %d", opt->force_chunk,
                        FD_CHUNK_QUANTUM);
        if (opt->force_kernel < FD_KERNEL_AUTO || opt->force_kernel > FD_KERNEL_MFMA)
            return fail(FD_ERR_INVALID_ARG, "unknown force_kernel %d", opt->force_kernel);
        if (opt->debug_checks != 0 && opt->debug_checks != 1)
            return fail(FD_ERR_INVALID_ARG, "fd_options.debug_checks must be 0 or 1 (got %d)", opt->debug_checks);
        if (opt->force_merge < FD_MERGE_AUTO || opt->force_merge > FD_MERGE_FUSED)
            return fail(FD_ERR_INVALID_ARG, "unknown force_merge %d", opt->force_merge);
        if (opt->force_launch < FD_LAUNCH_AUTO || opt->force_launch > FD_LAUNCH_PERSISTENT)
            return fail(FD_ERR_INVALID_ARG, "unknown force_launch %d", opt->force_launch);
    }
    return FD_OK;
}

// Whether a paged launch numbers its items (work list): sequence b has at most
// 1 + L_b / chunk splits, so a known total bounds the items by B + total / chunk.
// When the full (splits x sequences) grid would be more than twice that, the
// launch holds that many workgroups instead. An understated total_kv leaves
// items without a workgroup; their outputs become NaN.
// Splits of a sequence of `len` tokens: ceil(len / chunk) for a paged batch (the
// last split holds the remainder), max(1, floor(len / chunk)) for a contiguous
// cache (the last split also takes the remainder); at least one, so that a
// plan always has a split to hold an empty sequence's zeros.
long long splits_for(long long len, long long chunk, bool paged) {
    return paged ? std::max(1LL, (len + chunk - 1) / chunk) : std::max(1LL, len / chunk);
}

bool uses_work_list(int B, int max_len, long long total, bool total_known, long long chunk) {
    if (!total_known || B <= 1 || B > fd::kMaxListSeqs) return false;
    const long long splits = splits_for(max_len, chunk, true);
    const long long items = (long long)B + total / chunk;
    return (long long)B * splits >= 2 * items;
}

// Shared planner. `max_len` is the longest sequence, `total` the sum of the
// lengths (one sequence for contiguous decode), `page_size` 0 when contiguous.
fd_status make_plan(int B, int H, int Hkv, fd_dtype dtype, int max_len, long long total, bool total_known,
                    int page_size, int num_cus, const fd_options *opt, fd_plan *p) {
    const int G = H / Hkv;
    const int kernel = pick_kernel(dtype, G, opt ? opt->force_kernel : FD_KERNEL_AUTO);
    if (kernel < 0)
        return fail(FD_ERR_UNSUPPORTED, "the matrix-core kernel needs f16/bf16 and H/Hkv <= 16 or a multiple of 16");
    const int gt = kernel == FD_KERNEL_MFMA ? mfma_heads_per_group(G) : valu_heads_per_group(G, dtype);
    // MHA on the vector ALUs: adjacent KV heads share a workgroup so that each load
    // instruction reads their contiguous rows (512 B; 4 heads for 128-B E4M3 rows).
    int hp = 1;
    if (kernel == FD_KERNEL_VALU && G == 1) {
        hp = fd::is_fp8_cache(dtype) ? 4 : 2;
        while (hp > 1 && Hkv % hp != 0) hp /= 2;
    }
    const long long slices = (long long)(Hkv / hp) * (G / gt);

    long long chunk;
    if (opt && opt->force_chunk > 0) {
        chunk = opt->force_chunk;
    } else if (opt && opt->force_num_splits > 0) {
        // the largest quantum multiple not above max_len / n: about n splits
        const long long per = (long long)max_len / opt->force_num_splits;
        chunk = std::max<long long>(FD_CHUNK_QUANTUM, per / FD_CHUNK_QUANTUM * FD_CHUNK_QUANTUM);
    } else if (page_size > 0) {
        const double row_bytes = 2.0 * FD_HEAD_DIM * cache_elem_bytes(dtype) * hp;  // K + V of one token, per workgroup
        const double per_slot =
            (double)std::max(total, 1LL) * (Hkv / hp) * row_bytes / ((double)num_cus * kPagedSlotsPerCu);
        const double fixed_scale = fd::is_fp8_cache(dtype) ? kWgFixedFp8Scale : 1.0;
        auto balanced = [&](double fixed_bytes) {
            fixed_bytes *= fixed_scale;
            const double tokens = std::sqrt(2.0 * per_slot * fixed_bytes) / row_bytes;
            const long long c = 1LL << std::max(0L, std::lround(std::log2(std::max(tokens, 1.0))));  // nearest power of two
            return std::min<long long>(std::max<long long>(c, kMinChunk), kMaxChunk);
        };
        chunk = balanced(kWgFixedBytes);
        if (uses_work_list(B, max_len, total, total_known, chunk)) {
            const long long c = balanced(kWgFixedBytesList);
            if (uses_work_list(B, max_len, total, total_known, c)) chunk = c;
        }
    } else {
        // The splits that give the workgroups wanted (head slices x splits), then
        // the tokens per split: S / splits rounded down to a multiple of 16, so
        // that the fold gives exactly those splits and the last one holds fewer
        // than 16 x splits extra tokens. A grid just past a multiple of the CUs
        // would put two workgroups on a few CUs, whose halved bandwidth sets the
        // kernel's time: 283264 tokens of a GQA4 cache in 34 power-of-two splits
        // (272 workgroups) ran at 44% of peak, the same bytes on 256 workgroups
        // at 76%. A coarser rounding (64) left 100000 tokens with a last split
        // 1.55 times the others.
        const long long kv_bytes = std::max(total, 1LL) * Hkv * 2LL * FD_HEAD_DIM * cache_elem_bytes(dtype);
        const long long target = (long long)num_cus * target_wgs_per_cu(dtype, H == Hkv, kv_bytes);
        const long long want = std::max(1LL, target / slices);
        const long long per = std::max(1LL, std::max(total, 1LL) / want);
        chunk = per / kMinChunk * kMinChunk;
        chunk = std::min<long long>(std::max<long long>(chunk, kMinChunk), kMaxChunk);
    }
    // A paged split spans at most chunk tokens, i.e. at most (chunk - 1) / page_size
    // + 2 pages, and its slice of the block table must fit the LDS stage of
    // kMaxSplitPages entries.
    const long long page_cap =
        page_size > 0 ? (long long)(fd::kMaxSplitPages - 2) * page_size + 1 : (long long)1 << 40;
    if (page_size > 0) {
        const long long cap = page_cap / FD_CHUNK_QUANTUM * FD_CHUNK_QUANTUM;
        if (chunk > cap) {
            if (opt && opt->force_chunk > 0)
                return fail(FD_ERR_INVALID_ARG, "force_chunk %d: a split could span more than %d pages of %d tokens",
                            opt->force_chunk, fd::kMaxSplitPages, page_size);
            chunk = std::max<long long>(cap, FD_CHUNK_QUANTUM);
        }
    }
    const bool paged = page_size > 0;
    long long splits = splits_for(max_len, chunk, paged);
    if (splits > kMaxSplits) {
        chunk = ((long long)max_len + kMaxSplits - 1) / kMaxSplits;
        chunk = (chunk + FD_CHUNK_QUANTUM - 1) / FD_CHUNK_QUANTUM * FD_CHUNK_QUANTUM;
        if (chunk > page_cap)
            return fail(FD_ERR_UNSUPPORTED, "sequence of %d tokens needs more than %d splits", max_len, kMaxSplits);
        splits = splits_for(max_len, chunk, paged);
    }

    std::memset(p, 0, sizeof(*p));
    p->kernel = kernel;
    p->heads_per_group = gt;
    p->chunk = (int)chunk;
    p->num_splits = (int)splits;
    // Head slices vary fastest: workgroups go to the XCDs round-robin by linear
    // id, so this spreads every split index (and the empty tail splits of short
    // sequences) evenly over the XCDs.
    p->grid_x = (int)slices;
    p->grid_y = (int)splits;
    p->grid_z = B;
    p->threads = 256;
    p->kv_heads_per_group = hp;
    // Work list (uses_work_list): grid y numbers the items that exist.
    if (page_size > 0 && uses_work_list(B, max_len, total, total_known, chunk)) {
        p->work_list = 1;
        p->grid_y = (int)std::min((long long)B + total / chunk, (long long)B * splits);
        p->grid_z = 1;
    }
    p->head_slices = (int)slices;
    // Persistent paged launch: when the items would take more than one round of
    // resident workgroups, one workgroup per slot claims them instead (see
    // paged_items in fd_device.h). With one workgroup per item, slots emptied by
    // short items waited microseconds for the dispatcher and the XCDs, which get
    // workgroups round-robin, finished up to 20% apart on equal work.
    if (page_size > 0) {
        const int forced_launch = opt ? opt->force_launch : FD_LAUNCH_AUTO;
        const long long slots = (long long)num_cus * kPagedSlotsPerCu;
        const long long items = p->work_list ? (long long)p->grid_y : (long long)B * splits;
        const bool can = B <= fd::kMaxListSeqs;
        if (forced_launch == FD_LAUNCH_PERSISTENT && !can)
            return fail(FD_ERR_UNSUPPORTED, "a persistent launch numbers at most %d sequences", fd::kMaxListSeqs);
        const bool want = forced_launch == FD_LAUNCH_PERSISTENT ||
                          (forced_launch == FD_LAUNCH_AUTO && can && items * slices > slots);
        if (want) {
            p->persistent = 1;
            p->grid_x = (int)std::min(slots, items * slices);
            p->grid_y = 1;
            p->grid_z = 1;
        }
    }
    // Merge of the partials. A fused launch (contiguous caches only) needs a
    // counter per head slice in the workspace's head block and merges at most
    // kFusedMaxSplits splits in one workgroup. The merge kernel is the default:
    // on the 4k-token 32-head decode the fused step measured 16.4-16.6 us against
    // 15.1 us, and on the 512-token 8-head fp32 decode 8.3-8.4 us against 6.3-7.5
    // us. Its tail (partial stores written through to memory, a wait for them, a
    // counter round trip, the reads of the last workgroup) is three dependent
    // memory round trips on every workgroup's critical path, while the merge
    // kernel after the split kernel adds about 2 us to a step.
    const int forced_merge = opt ? opt->force_merge : FD_MERGE_AUTO;
    const bool fusable = page_size == 0 && splits <= fd::kFusedMaxSplits && slices <= fd::kFusedCounters &&
                         gt * hp <= fd::kFusedMaxHeads && (long long)gt * hp * splits <= fd::kFusedMaxRows;
    if (splits <= 1) {
        p->merge = 0;
    } else if (forced_merge == FD_MERGE_FUSED) {
        if (!fusable)
            return fail(FD_ERR_UNSUPPORTED, "this plan cannot merge in its last workgroups (a contiguous cache "
                        "of at most %d splits and %d (head, split) rows per workgroup: %lld splits, %lld rows%s)",
                        fd::kFusedMaxSplits, fd::kFusedMaxRows, splits, (long long)gt * hp * splits,
                        page_size > 0 ? ", paged" : "");
        p->merge = FD_MERGE_FUSED;
    } else if (forced_merge == FD_MERGE_KERNEL) {
        p->merge = FD_MERGE_KERNEL;
    } else {
        p->merge = FD_MERGE_KERNEL;
    }
    if (p->merge) {
        const size_t rows = (size_t)B * H * splits;
        const size_t o_bytes = rows * FD_HEAD_DIM * sizeof(float);
        p->ws_o_offset = FD_WS_COUNTER_BYTES;
        p->ws_lse_offset = p->ws_o_offset + (o_bytes + 255) / 256 * 256;
        p->workspace_bytes = p->ws_lse_offset + rows * sizeof(float);
    } else if (p->persistent) {
        p->ws_o_offset = FD_WS_COUNTER_BYTES;
        p->workspace_bytes = FD_WS_COUNTER_BYTES;  // the claim counters
    }
    // Debug record of a paged call: four ints after the partials.
    if (page_size > 0 && opt && opt->debug_checks) {
        p->ws_err_offset = (p->workspace_bytes + 255) / 256 * 256;
        p->workspace_bytes = p->ws_err_offset + kErrRecordBytes;
    }
    return FD_OK;
}

fd_status resolve_cus(int *num_cus) {
    if (*num_cus > 0) return FD_OK;
    if (*num_cus < 0) return fail(FD_ERR_INVALID_ARG, "num_cus must be >= 0");
    const int n = fd_device_num_cus();
    if (n < 1) return fail(FD_ERR_DEVICE, "cannot query the compute units of the current device");
    *num_cus = n;
    return FD_OK;
}

// Reads back the debug record after the launches (waits for the stream) and turns
// a recorded violation into FD_ERR_BAD_DATA.
fd_status debug_verdict(const int32_t *err, hipStream_t stream) {
    int32_t rec[4] = {0, 0, 0, 0};
    hipError_t e = hipMemcpyAsync(rec, err, sizeof(rec), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return fail(FD_ERR_LAUNCH, "reading the debug record: %s", hipGetErrorString(e));
    if (rec[0] == fd::kBadTableEntry)
        return fail(FD_ERR_BAD_DATA, "block_table[%d][%d] = %d is outside [0, num_pages)", rec[1], rec[2], rec[3]);
    if (rec[0] == fd::kBadSeqLen)
        return fail(FD_ERR_BAD_DATA, "seq_lens[%d] = %d is outside [0, min(max_seq_len, max_blocks * page_size)]",
                    rec[1], rec[3]);
    if (rec[0] != 0) return fail(FD_ERR_BAD_DATA, "debug record holds unknown kind %d", rec[0]);
    return FD_OK;
}

fd_status run(const fd_plan &plan, fd_dtype dtype, bool paged, fd::SplitArgs &a, fd::MergeArgs &m, int B,
              void *ws, size_t ws_bytes, const fd_options *opt, hipStream_t stream, bool static_ws = false) {
    if (plan.workspace_bytes > 0) {
        if (static_ws && ws_bytes < plan.workspace_bytes)
            return fail(FD_ERR_WORKSPACE,
                        "this call needs %zu bytes of workspace, more than the library's static scratch of %zu "
                        "bytes: pass a larger fd_options.force_chunk (fewer splits), or call fd_paged_decode "
                        "with a workspace", plan.workspace_bytes, ws_bytes);
        if (ws == nullptr || ws_bytes < plan.workspace_bytes)
            return fail(FD_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given%s", plan.workspace_bytes, ws_bytes,
                        ws == nullptr ? " (NULL)" : "");
        if (!aligned16(ws)) return fail(FD_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    }
    const bool debug = paged && opt && opt->debug_checks;
    a.err = debug ? reinterpret_cast<int *>(reinterpret_cast<char *>(ws) + plan.ws_err_offset) : nullptr;
    if (debug) {
        const hipError_t e = hipMemsetAsync(a.err, 0, kErrRecordBytes, stream);
        if (e != hipSuccess) return fail(FD_ERR_LAUNCH, "clearing the debug record: %s", hipGetErrorString(e));
    }
    if (plan.merge) {
        a.ws_o = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + plan.ws_o_offset);
        a.ws_lse = reinterpret_cast<float *>(reinterpret_cast<char *>(ws) + plan.ws_lse_offset);
    } else {
        a.ws_o = nullptr;
        a.ws_lse = nullptr;
    }
    const bool fused = plan.merge == FD_MERGE_FUSED;
    a.persistent = plan.persistent;
    a.slices = plan.head_slices;
    a.counters = plan.workspace_bytes > 0 ? reinterpret_cast<unsigned *>(ws) : nullptr;
    a.chunk = plan.chunk;
    a.num_splits = plan.num_splits;
    a.B = B;
    a.work_list = plan.work_list;
    a.grid_items = plan.grid_y;
    fd::LaunchShape shape{dim3(plan.grid_x, plan.grid_y, plan.grid_z), dim3(plan.threads)};

    hipEvent_t ev0 = opt ? reinterpret_cast<hipEvent_t>(opt->split_begin_event) : nullptr;
    hipEvent_t ev1 = opt ? reinterpret_cast<hipEvent_t>(opt->split_end_event) : nullptr;
    a.heads_per_wg = plan.heads_per_group;
    // 16-token blocks stay inside one page when pages hold at least 16 tokens.
    const int mode = !paged ? fd::kContig : ((1 << a.page_shift) >= 16 ? fd::kPagedBlock : fd::kPagedRow);
    const bool persist = plan.persistent != 0;
    hipError_t e = plan.kernel == FD_KERNEL_MFMA
                       ? fd::launch_split_mfma(dtype, plan.heads_per_group, mode, persist, fused, shape, a, stream,
                                               ev0, ev1)
                       : fd::launch_split_valu(dtype, plan.heads_per_group, plan.kv_heads_per_group, mode, persist,
                                               fused, shape, a, stream, ev0, ev1);
    if (e != hipSuccess) return fail(FD_ERR_LAUNCH, "split kernel launch: %s", hipGetErrorString(e));
    if (plan.merge == FD_MERGE_KERNEL) {
        m.ws_o = a.ws_o;
        m.ws_lse = a.ws_lse;
        m.chunk = plan.chunk;
        m.num_splits = plan.num_splits;
        // Contiguous grid (slices, splits): workgroup (x, y) is dispatched to XCD
        // (y * slices + x) mod 8 = x mod 8 when slices is a multiple of 8.
        m.xcd_group = (!paged && plan.grid_x % 8 == 0 && m.H % 8 == 0 && plan.grid_z == 1) ? m.H / plan.grid_x : 0;
        e = fd::launch_merge(fd::query_dtype(dtype), paged, B, m, stream);
        if (e != hipSuccess) return fail(FD_ERR_LAUNCH, "merge kernel launch: %s", hipGetErrorString(e));
    }
    if (debug) return debug_verdict(a.err, stream);
    return FD_OK;
}

}  // namespace

extern "C" {

int fd_device_num_cus(void) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if ((int)g_cu_cache.size() <= dev) g_cu_cache.resize(dev + 1, 0);
    if (g_cu_cache[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return -1;
        g_cu_cache[dev] = n;
    }
    return g_cu_cache[dev];
}

fd_status fd_decode_plan(int H, int Hkv, int S, int D, fd_dtype dtype, int num_cus, const fd_options *opt,
                         fd_plan *out) {
    if (!out) return fail(FD_ERR_INVALID_ARG, "out is NULL");
    fd_status s = check_common(1, H, Hkv, D, dtype, opt);
    if (s != FD_OK) return s;
    if (S < 0) return fail(FD_ERR_INVALID_ARG, "S must be >= 0 (got %d)", S);
    if ((s = resolve_cus(&num_cus)) != FD_OK) return s;
    return make_plan(1, H, Hkv, dtype, S, S, true, 0, num_cus, opt, out);
}

fd_status fd_paged_plan(int B, int H, int Hkv, int D, fd_dtype dtype, int page_size, int max_seq_len,
                        long long total_kv, int num_cus, const fd_options *opt, fd_plan *out) {
    if (!out) return fail(FD_ERR_INVALID_ARG, "out is NULL");
    fd_status s = check_common(B, H, Hkv, D, dtype, opt);
    if (s != FD_OK) return s;
    if (ilog2_exact(page_size) < 0 || page_size > 1024)
        return fail(FD_ERR_UNSUPPORTED, "page_size %d is not a power of two in [1, 1024]", page_size);
    if (max_seq_len < 0) return fail(FD_ERR_INVALID_ARG, "max_seq_len must be >= 0");
    if ((s = resolve_cus(&num_cus)) != FD_OK) return s;
    const long long total = total_kv > 0 ? total_kv : (long long)B * max_seq_len;
    return make_plan(B, H, Hkv, dtype, max_seq_len, total, total_kv > 0, page_size, num_cus, opt, out);
}

fd_status fd_decode_workspace_size(int H, int Hkv, int S, int D, fd_dtype dtype, int num_cus,
                                   const fd_options *opt, size_t *bytes) {
    if (!bytes) return fail(FD_ERR_INVALID_ARG, "bytes is NULL");
    fd_plan p;
    const fd_status s = fd_decode_plan(H, Hkv, S, D, dtype, num_cus, opt, &p);
    if (s == FD_OK) *bytes = p.workspace_bytes;
    return s;
}

fd_status fd_paged_workspace_size(int B, int H, int Hkv, int D, fd_dtype dtype, int page_size, int max_seq_len,
                                  long long total_kv, int num_cus, const fd_options *opt, size_t *bytes) {
    if (!bytes) return fail(FD_ERR_INVALID_ARG, "bytes is NULL");
    fd_plan p;
    const fd_status s = fd_paged_plan(B, H, Hkv, D, dtype, page_size, max_seq_len, total_kv, num_cus, opt, &p);
    if (s == FD_OK) *bytes = p.workspace_bytes;
    return s;
}

}  // extern "C"

namespace {

fd_status check_scales(float k_scale, float v_scale) {
    if (!std::isfinite(k_scale) || !std::isfinite(v_scale))
        return fail(FD_ERR_INVALID_ARG, "k_scale and v_scale must be finite");
    return FD_OK;
}

// The kernels take the scores in the log2 domain: scale * k_scale * log2(e) must
// be a finite float (an infinite one would turn every exponent into inf - inf).
fd_status check_score_scale(float scale, float k_scale) {
    if (!std::isfinite(scale) || !std::isfinite(scale * k_scale * fd::kLog2eHost))
        return fail(FD_ERR_INVALID_ARG, "scale must be finite (scale * k_scale * log2(e) = %g)",
                    (double)(scale * k_scale * fd::kLog2eHost));
    return FD_OK;
}

fd_status decode_impl(const void *q, const void *k, const void *v, void *o, int H, int Hkv, int S, int D,
                      fd_dtype dtype, float scale, float k_scale, float v_scale, void *ws, size_t ws_bytes,
                      const fd_options *opt, void *stream) {
    fd_status s = check_common(1, H, Hkv, D, dtype, opt);
    if (s != FD_OK) return s;
    if ((s = check_score_scale(scale, k_scale)) != FD_OK) return s;
    if (S < 0) return fail(FD_ERR_INVALID_ARG, "S must be >= 0 (got %d)", S);
    if (!q || !o || (S > 0 && (!k || !v))) return fail(FD_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(FD_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    fd_plan plan;
    if ((s = fd_decode_plan(H, Hkv, S, D, dtype, 0, opt, &plan)) != FD_OK) return s;

    fd::SplitArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = o;
    a.H = H;
    a.Hkv = Hkv;
    a.G = H / Hkv;
    a.max_len = S;
    a.scale_log2 = scale * k_scale * fd::kLog2eHost;
    a.v_scale = v_scale;
    fd::MergeArgs m{};
    m.out = o;
    m.H = H;
    m.max_len = S;
    return run(plan, dtype, false, a, m, 1, ws, ws_bytes, opt, reinterpret_cast<hipStream_t>(stream));
}

fd_status paged_impl(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_table,
                     const int32_t *seq_lens, int page_size, void *o, float scale, float k_scale, float v_scale,
                     int B, int H, int Hkv, int D, int num_pages, int max_blocks, int max_seq_len, long long total_kv,
                     fd_dtype dtype, void *ws, size_t ws_bytes, const fd_options *opt, void *stream,
                     bool static_ws = false) {
    fd_status s = check_common(B, H, Hkv, D, dtype, opt);
    if (s != FD_OK) return s;
    if ((s = check_score_scale(scale, k_scale)) != FD_OK) return s;
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !o)
        return fail(FD_ERR_INVALID_ARG, "q, k_cache, v_cache, block_table, seq_lens and o must not be NULL");
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
        return fail(FD_ERR_INVALID_ARG, "q, k_cache, v_cache and o must be 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
        return fail(FD_ERR_INVALID_ARG, "block_table and seq_lens must be 4-byte aligned");
    if (num_pages < 1 || max_blocks < 1) return fail(FD_ERR_INVALID_ARG, "num_pages and max_blocks must be >= 1");
    const int shift = ilog2_exact(page_size);
    if (shift < 0 || page_size > 1024)
        return fail(FD_ERR_UNSUPPORTED, "page_size %d is not a power of two in [1, 1024]", page_size);
    if (max_seq_len < 0) return fail(FD_ERR_INVALID_ARG, "max_seq_len must be >= 0");
    // Every length is clamped to what the table can address.
    const long long addressable = (long long)max_blocks * page_size;
    const int eff_max = (int)std::min<long long>(max_seq_len, addressable);
    fd_plan plan;
    if ((s = fd_paged_plan(B, H, Hkv, D, dtype, page_size, eff_max, total_kv, 0, opt, &plan)) != FD_OK) return s;

    fd::SplitArgs a{};
    a.q = q;
    a.k = k_cache;
    a.v = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.out = o;
    a.H = H;
    a.Hkv = Hkv;
    a.G = H / Hkv;
    a.max_len = eff_max;
    a.page_shift = shift;
    a.max_blocks = max_blocks;
    a.num_pages = num_pages;
    a.scale_log2 = scale * k_scale * fd::kLog2eHost;
    a.v_scale = v_scale;
    fd::MergeArgs m{};
    m.seq_lens = seq_lens;
    m.out = o;
    m.H = H;
    m.max_len = eff_max;
    return run(plan, dtype, true, a, m, B, ws, ws_bytes, opt, reinterpret_cast<hipStream_t>(stream), static_ws);
}

// Static scratch of fd_paged_decode_noalloc: a device array every GPU the
// library runs on holds until the process ends. In host code `scratch` only
// names the array (it is not a device address): its address on the current
// device comes from hipGetSymbolAddress, taken once per device and kept in
// g_scratch_ptr, and only that pointer is passed to kernels.
static __device__ __align__(256) unsigned char scratch[FD_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
std::vector<void *> g_scratch_ptr;

__global__ void zero_words_kernel(unsigned *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

// The scratch address on the current device. The first call on a device looks it
// up and clears the counter block at its head with a fill kernel on `stream`
// (a kernel, not a memset, so that the call may be captured into a graph).
fd_status scratch_of_current_device(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(FD_ERR_DEVICE, "no current HIP device");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return fail(FD_ERR_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, stream, reinterpret_cast<unsigned *>(p),
                           (int)(FD_WS_COUNTER_BYTES / sizeof(unsigned)));
        const hipError_t le = hipGetLastError();
        if (le != hipSuccess) return fail(FD_ERR_LAUNCH, "clearing the scratch counters: %s", hipGetErrorString(le));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return FD_OK;
}

}  // namespace

extern "C" {

fd_status fd_paged_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *seq_lens, int page_size, void *o,
                                  float scale, int B, int H, int Hkv, int D, int num_pages, int max_blocks,
                                  int max_seq_len, long long total_kv, fd_dtype dtype, const fd_options *opt,
                                  void *stream) {
    if (fd::is_fp8_cache(dtype)) return fail(FD_ERR_UNSUPPORTED, "FP8 KV caches go through fd_paged_decode_fp8kv");
    void *ws = nullptr;
    const fd_status s = scratch_of_current_device(reinterpret_cast<hipStream_t>(stream), &ws);
    if (s != FD_OK) return s;
    return paged_impl(q, k_cache, v_cache, block_table, seq_lens, page_size, o, scale, 1.f, 1.f, B, H, Hkv, D,
                      num_pages, max_blocks, max_seq_len, total_kv, dtype, ws, FD_NOALLOC_SCRATCH_BYTES, opt, stream,
                      true);
}

fd_status fd_decode(const void *q, const void *k, const void *v, void *o, int H, int Hkv, int S, int D,
                    fd_dtype dtype, float scale, void *ws, size_t ws_bytes, const fd_options *opt, void *stream) {
    if (fd::is_fp8_cache(dtype)) return fail(FD_ERR_UNSUPPORTED, "FP8 KV caches go through fd_decode_fp8kv");
    return decode_impl(q, k, v, o, H, Hkv, S, D, dtype, scale, 1.f, 1.f, ws, ws_bytes, opt, stream);
}

fd_status fd_decode_fp8kv(const void *q, const void *k, const void *v, void *o, int H, int Hkv, int S, int D,
                          fd_dtype dtype, float scale, float k_scale, float v_scale, void *ws, size_t ws_bytes,
                          const fd_options *opt, void *stream) {
    if (!fd::is_fp8_cache(dtype))
        return fail(FD_ERR_UNSUPPORTED, "fd_decode_fp8kv takes FD_DTYPE_F16_KV_E4M3 or FD_DTYPE_BF16_KV_E4M3");
    fd_status s = check_scales(k_scale, v_scale);
    if (s != FD_OK) return s;
    return decode_impl(q, k, v, o, H, Hkv, S, D, dtype, scale, k_scale, v_scale, ws, ws_bytes, opt, stream);
}

fd_status fd_paged_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_table,
                          const int32_t *seq_lens, int page_size, void *o, float scale, int B, int H, int Hkv, int D,
                          int num_pages, int max_blocks, int max_seq_len, long long total_kv, fd_dtype dtype,
                          void *ws, size_t ws_bytes, const fd_options *opt, void *stream) {
    if (fd::is_fp8_cache(dtype)) return fail(FD_ERR_UNSUPPORTED, "FP8 KV caches go through fd_paged_decode_fp8kv");
    return paged_impl(q, k_cache, v_cache, block_table, seq_lens, page_size, o, scale, 1.f, 1.f, B, H, Hkv, D,
                      num_pages, max_blocks, max_seq_len, total_kv, dtype, ws, ws_bytes, opt, stream);
}

fd_status fd_paged_decode_fp8kv(const void *q, const void *k_cache, const void *v_cache, const int32_t *block_table,
                                const int32_t *seq_lens, int page_size, void *o, float scale, float k_scale,
                                float v_scale, int B, int H, int Hkv, int D, int num_pages, int max_blocks,
                                int max_seq_len, long long total_kv, fd_dtype dtype, void *ws, size_t ws_bytes,
                                const fd_options *opt, void *stream) {
    if (!fd::is_fp8_cache(dtype))
        return fail(FD_ERR_UNSUPPORTED, "fd_paged_decode_fp8kv takes FD_DTYPE_F16_KV_E4M3 or FD_DTYPE_BF16_KV_E4M3");
    fd_status s = check_scales(k_scale, v_scale);
    if (s != FD_OK) return s;
    return paged_impl(q, k_cache, v_cache, block_table, seq_lens, page_size, o, scale, k_scale, v_scale, B, H, Hkv,
                      D, num_pages, max_blocks, max_seq_len, total_kv, dtype, ws, ws_bytes, opt, stream);
}

size_t fd_prefill_workspace_size(int B, int N, int Hkv, int D, fd_dtype dtype) {
    if (dtype != FD_DTYPE_BF16 || B <= 0 || N <= 0 || Hkv <= 0 || D != 128) return 0;
    if ((long long)B * Hkv * ((N + 63) / 64) > INT_MAX) return 0;  // fd_prefill refuses these sizes
    return fd::prefill_workspace_bytes(B, N, Hkv);
}

fd_status fd_prefill(const void *q, const void *k, const void *v, void *o, int B, int N, int H, int Hkv, int D,
                     fd_dtype dtype, float scale, int causal, void *ws, size_t ws_bytes, const fd_options *opt,
                     void *stream) {
    fd_status s = check_common(B, H, Hkv, D, dtype, opt);
    if (s != FD_OK) return s;
    if (dtype != FD_DTYPE_F16 && dtype != FD_DTYPE_BF16)
        return fail(FD_ERR_UNSUPPORTED, "prefill runs on the matrix cores: f16 or bf16 only");
    if (N < 0) return fail(FD_ERR_INVALID_ARG, "N must be >= 0 (got %d)", N);
    if (N > (1 << 30)) return fail(FD_ERR_UNSUPPORTED, "N must be <= 2^30 (got %d)", N);
    if (!std::isfinite(scale)) return fail(FD_ERR_INVALID_ARG, "scale must be finite");
    if (B > 65535 || H > 65535) return fail(FD_ERR_UNSUPPORTED, "B and H must be <= 65535");
    if ((long long)B * H * ((N + 63) / 64) > INT_MAX)
        return fail(FD_ERR_UNSUPPORTED, "B * H * ceil(N / 64) must fit in 31 bits");
    if (N == 0) return FD_OK;
    if (!q || !k || !v || !o) return fail(FD_ERR_INVALID_ARG, "q, k, v and o must not be NULL");
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
        return fail(FD_ERR_INVALID_ARG, "q, k, v and o must be 16-byte aligned");
    // The workspace serves bf16 only (the f16 copy of V); f16 ignores it.
    if (dtype != FD_DTYPE_BF16) ws = nullptr;
    if (ws) {
        const size_t need = fd::prefill_workspace_bytes(B, N, Hkv);
        if (ws_bytes < need)
            return fail(FD_ERR_WORKSPACE, "prefill workspace is %zu bytes, %zu needed", ws_bytes, need);
        if (!aligned16(ws)) return fail(FD_ERR_INVALID_ARG, "the prefill workspace must be 16-byte aligned");
    }
    fd::PrefillArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.B = B;
    a.N = N;
    a.H = H;
    a.Hkv = Hkv;
    a.G = H / Hkv;
    a.causal = causal ? 1 : 0;
    a.scale_log2 = scale * fd::kLog2eHost;
    // The kernel needs a nonzero factor (a masked score must stay -inf after
    // scaling); with the least normal float every unmasked score still scales to
    // exactly 0 in exp2, as with a zero scale.
    if (a.scale_log2 == 0.f) a.scale_log2 = FLT_MIN;
    hipEvent_t ev0 = opt ? reinterpret_cast<hipEvent_t>(opt->split_begin_event) : nullptr;
    hipEvent_t ev1 = opt ? reinterpret_cast<hipEvent_t>(opt->split_end_event) : nullptr;
    const hipError_t e = fd::launch_prefill(dtype, a, ws, reinterpret_cast<hipStream_t>(stream), ev0, ev1);
    if (e != hipSuccess) return fail(FD_ERR_LAUNCH, "prefill kernel launch: %s", hipGetErrorString(e));
    return FD_OK;
}

const char *fd_status_string(fd_status s) {
    switch (s) {
        case FD_OK: return "FD_OK";
        case FD_ERR_INVALID_ARG: return "FD_ERR_INVALID_ARG";
        case FD_ERR_UNSUPPORTED: return "FD_ERR_UNSUPPORTED";
        case FD_ERR_WORKSPACE: return "FD_ERR_WORKSPACE";
        case FD_ERR_DEVICE: return "FD_ERR_DEVICE";
        case FD_ERR_LAUNCH: return "FD_ERR_LAUNCH";
        case FD_ERR_BAD_DATA: return "FD_ERR_BAD_DATA";
    }
    return "FD_ERR_UNKNOWN";
}

const char *fd_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"

// fd_internal.h -- argument blocks shared by the C-ABI layer and the kernel
// launchers. Not part of the public interface.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fd.h"

namespace fd {

// Most physical pages one split may touch: the paged split kernel stages the
// split's block-table slice in LDS. A split spans up to 2*chunk - 1 tokens, so
// the planner keeps (2*chunk - 2) / page_size + 2 within this bound.
constexpr int kMaxSplitPages = 1024;

constexpr float kLog2eHost = 1.4426950408889634f;  // log2(e), folded into the scale on the host

// How a split kernel addresses K/V rows (see KvAddr in fd_device.h).
enum AddrMode { kContig = 0, kPagedBlock = 1, kPagedRow = 2 };

struct SplitArgs {
    const void *q;          // [B, H, D]
    const void *k;          // contiguous [S, Hkv, D] or cache [num_pages, page_size, Hkv, D]
    const void *v;
    const int32_t *block_table;  // [B, max_blocks] (paged)
    const int32_t *seq_lens;     // [B] (paged)
    float *ws_o;            // [B, H, num_splits, D]
    float *ws_lse;          // [B, H, num_splits]
    void *out;              // [B, H, D]
    int H, Hkv, G;          // G = H / Hkv
    int heads_per_wg;       // query heads of one KV head computed by one workgroup
    int max_len;            // contiguous: S; paged: clamp bound for seq_lens
    int chunk;              // split stride (a sequence's last split also takes the remainder)
    int num_splits;
    int page_shift;         // log2(page_size)
    int max_blocks;
    int num_pages;
    float scale_log2;       // scale * k_scale * log2(e)
    float v_scale;          // dequantisation scale of V (1 unless the cache is FP8)
    int B;                  // sequences (paged)
    int work_list;          // 1: grid y numbers the splits that hold tokens (paged; see the split kernels)
    int grid_items;         // grid y when work_list is set
    int *err;               // paged with debug_checks: 4-int error record (kind, sequence, index, value); else NULL
    unsigned *counters;     // workspace counter block: fused-merge counters per head slice at its
                            // head, the persistent launch's claim and exit counters at its end; all
                            // zero between calls
    int slices;             // head slices per sequence (grid x of a one-item-per-workgroup launch)
    int persistent;         // paged: 1 = one workgroup per resident slot, claiming items (see fd_device.h)
};

// Fused launches: splits per sequence and heads per workgroup one workgroup
// merges at the end, and counters at the head of every workspace.
constexpr int kFusedMaxSplits = 32;
constexpr int kFusedMaxHeads = 16;
constexpr int kFusedMaxRows = 64;  // heads x splits one workgroup merges (4 x 32 or 16 x 4, ...)
constexpr int kWsCounters = FD_WS_COUNTER_BYTES / 4;
// Persistent launch, at the end of the block, each counter on a 256-byte line of
// its own: the claim counter, the count of exit groups done, and one exit counter
// per group of workgroups (blockIdx.x % kExitGroups, its XCD).
constexpr int kExitGroups = 8;
constexpr int kQueueStride = 64;  // words between two counters
constexpr int kQueueBase = kWsCounters - (kExitGroups + 2) * kQueueStride;
constexpr int kFusedCounters = kQueueBase;  // fused-merge counters available at the head of the block

// Kinds of the debug error record.
enum BadData { kBadTableEntry = 1, kBadSeqLen = 2 };

// Sequences a work-list launch can hold (its per-sequence offsets live in LDS).
constexpr int kMaxListSeqs = 1024;

// Query/output dtype of a call (FP8-cache codes map to their query type).
inline fd_dtype query_dtype(fd_dtype d) {
    if (d == FD_DTYPE_F16_KV_E4M3) return FD_DTYPE_F16;
    if (d == FD_DTYPE_BF16_KV_E4M3) return FD_DTYPE_BF16;
    return d;
}

inline bool is_fp8_cache(fd_dtype d) { return d == FD_DTYPE_F16_KV_E4M3 || d == FD_DTYPE_BF16_KV_E4M3; }

struct MergeArgs {
    const float *ws_o;
    const float *ws_lse;
    const int32_t *seq_lens;  // paged only
    void *out;
    int H;
    int max_len;              // contiguous: S; paged: clamp bound for seq_lens
    int chunk;
    int num_splits;
    // > 0: head h of the split grid's slice h / xcd_group ran on XCD (slice mod 8);
    // workgroup i of the merge takes a head of slice = i mod 8 (mod 8), so it reads
    // partials its XCD's L2 may still hold. 0: workgroup i takes head i.
    int xcd_group;
};

struct LaunchShape {
    dim3 grid;
    dim3 block;
};

// Each returns hipSuccess or the launch error. `gt` = query heads per KV head in a
// workgroup, `hp` = adjacent KV heads per workgroup (vector-ALU kernel, MHA),
// `mode` = AddrMode of fd_device.h (contiguous, paged by 16-token block, paged by row);
// `persist` (paged modes): one workgroup per resident slot claiming items;
// `fused` (contiguous only): the last workgroup of each head slice merges.
// `start`/`stop` (may be NULL) are timestamped by the dispatch itself at the
// kernel's start and end (hipExtLaunchKernel), so they time the kernel alone.
hipError_t launch_split_valu(fd_dtype dtype, int gt, int hp, int mode, bool persist, bool fused,
                             const LaunchShape &shape, const SplitArgs &a, hipStream_t stream, hipEvent_t start,
                             hipEvent_t stop);
hipError_t launch_split_mfma(fd_dtype dtype, int gt, int mode, bool persist, bool fused, const LaunchShape &shape,
                             const SplitArgs &a, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

// Launch through hipExtLaunchKernel when events are given, else hipLaunchKernel.
inline hipError_t launch_timed(const void *fn, const LaunchShape &s, void **args, hipStream_t st, hipEvent_t start,
                               hipEvent_t stop) {
    if (start || stop) return hipExtLaunchKernel(fn, s.grid, s.block, args, 0, st, start, stop, 0);
    return hipLaunchKernel(fn, s.grid, s.block, args, 0, st);
}
hipError_t launch_merge(fd_dtype dtype, bool paged, int B, const MergeArgs &a, hipStream_t stream);

// Prefill: q, o [B, N, H, D]; k, v [B, N, Hkv, D].
// bf16 prefill with a workspace: V is first converted to an f16 copy (exact for
// |v| < 65536), with one flag byte per chunk of a sequence's V rows saying
// whether some value did not fit. Each sequence owns a row of kPrefillFlagRow
// flag bytes, of which the first flag_chunks are written.
constexpr int kPrefillFlagRow = 1024;
constexpr int kPrefillConvMinRows = 128;  // 256-byte V rows per conversion workgroup, at least
enum PrefillFlagMode : int {
    kPrefillNoFlags = 0,       // run every sequence
    kPrefillRunIfClean = 1,    // the f16-V kernel: skip sequences whose V did not convert
    kPrefillRunIfFlagged = 2,  // the split-P kernel after it: run only those sequences
};

struct PrefillArgs {
    const void *q, *k, *v;  // v: the caller's V, or its f16 copy (kPrefillRunIfClean)
    void *o;
    int B, N, H, Hkv, G;    // G = H / Hkv
    int causal;             // 1: query i sees keys 0 .. i
    int q_tiles;            // query tiles (set by the launcher)
    float scale_log2;       // scale * log2(e)
    const uint8_t *flags;   // B rows of kPrefillFlagRow bytes (flag modes 1 and 2)
    int flag_chunks;        // flags written per row
    int flag_mode;          // PrefillFlagMode
};

// Workspace bytes of the bf16 f16-V path: the f16 copy of V, then the flag rows.
size_t prefill_workspace_bytes(int B, int N, int Hkv);

// f16 and bf16 without a workspace: one kernel. bf16 with a workspace (at
// least prefill_workspace_bytes): conversion, the f16-V kernel, and the
// split-P kernel for the sequences that did not convert. start / stop (may be
// null) bracket the kernel that does the attention of the clean sequences.
hipError_t launch_prefill(fd_dtype dtype, const PrefillArgs &a, void *ws, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop);

}  // namespace fd

/*
 * fd.h -- split-KV ("Flash-Decoding") single-query decode attention for AMD
 * Instinct MI355X (gfx950). C ABI: plain pointers, sizes and status codes.
 *
 * What is computed. For every sequence b and query head h, with KV head
 * g = h / (H / Hkv) (consecutive query heads share one KV head, as in the GQA
 * paged decode kernel of "FlashAttention 与推理算子", section "一个分页 decode
 * attention kernel（支持 GQA）") and the L_b keys and values of that head:
 *
 *     s_t = scale * q[b,h,:] . k[t,g,:]          t = 0 .. L_b - 1
 *     o[b,h,:] = sum_t softmax(s)_t * v[t,g,:]
 *
 * i.e. S = Q K^T * scale, P = softmax(S), O = P V for one query row ("Flash
 * Attention 与推理算子", section "标准注意力的问题"). The KV sequence is cut
 * into splits of `chunk` tokens, the last split also taking the remainder
 * (see the workspace layout below); a first kernel computes each split's
 * normalised output and log-sum-exp with an online softmax, a second merges
 * the splits by log-sum-exp ("[CUDA 优化实战] 纯手搓 flash decoding sm120",
 * sections "1. flash decoding" and "2. kernel 实现细节"; "FlashAttention 与
 * 推理算子", section "decode 阶段的并行：Flash-Decoding 与 split-K"). When one
 * split covers the longest sequence the first kernel writes o directly and no
 * merge runs. The result does not depend on the split count beyond rounding.
 *
 * Conventions shared by every call:
 *   - All tensor pointers are DEVICE memory owned by the caller, contiguous
 *     row-major and 16-byte aligned. q, k, v and o share one dtype;
 *     accumulation is fp32; o is rounded to its dtype to nearest-even.
 *   - Calls are asynchronous on `stream` (a hipStream_t, NULL = the null
 *     stream): no synchronisation, no allocation, no hidden state except a
 *     cached compute-unit count per device. Thread-safe. Calls that share a
 *     workspace must not overlap.
 *   - Head dimension D must be 128 (FD_HEAD_DIM).
 *   - Errors are returned as fd_status; nothing is launched when a host-side
 *     check fails. fd_last_error() holds a message for the calling thread.
 */
#ifndef FD_H_
#define FD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FD_HEAD_DIM 128
#define FD_CHUNK_QUANTUM 64 /* a forced chunk must be a positive multiple of this */
#define FD_WS_COUNTER_BYTES 16384 /* counter block at the head of every workspace (see the layout below) */
#define FD_NOALLOC_SCRATCH_BYTES (64u << 20) /* the static scratch of fd_paged_decode_noalloc, per GPU */

typedef enum fd_dtype {
    FD_DTYPE_F32 = 0,
    FD_DTYPE_F16 = 1,
    FD_DTYPE_BF16 = 2,
    /* q and o in f16/bf16; K and V stored as OCP FP8 E4M3 codes (1 byte each)
     * with per-tensor dequantisation scales: only for the *_fp8kv calls and
     * their plans. */
    FD_DTYPE_F16_KV_E4M3 = 3,
    FD_DTYPE_BF16_KV_E4M3 = 4
} fd_dtype;

typedef enum fd_status {
    FD_OK = 0,
    FD_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, H % Hkv != 0, bad option */
    FD_ERR_UNSUPPORTED = 2, /* D != 128, page_size not a power of two in [1, 1024], dtype not valid for the call */
    FD_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than fd_plan.workspace_bytes */
    FD_ERR_DEVICE = 4,      /* no current HIP device / attribute query failed */
    FD_ERR_LAUNCH = 5,      /* a kernel launch or event record returned an error */
    FD_ERR_BAD_DATA = 6     /* debug_checks only: a block-table entry or sequence length that the
                               kernels read on the device was out of range (see fd_options) */
} fd_status;

enum {
    FD_MERGE_AUTO = 0,   /* planner's choice */
    FD_MERGE_KERNEL = 1, /* a second kernel merges the split partials */
    FD_MERGE_FUSED = 2   /* contiguous caches: the last workgroup of each head slice merges them: one launch */
};

enum {
    FD_LAUNCH_AUTO = 0,       /* planner's choice */
    FD_LAUNCH_GRID = 1,       /* paged: one workgroup per (head slice, split, sequence) */
    FD_LAUNCH_PERSISTENT = 2  /* paged: one workgroup per resident slot, each claiming items in turn */
};

enum {
    FD_KERNEL_AUTO = 0, /* planner's choice */
    FD_KERNEL_VALU = 1, /* vector-ALU split kernel (any head group, every dtype) */
    FD_KERNEL_MFMA = 2  /* matrix-core split kernel (f16/bf16, H/Hkv <= 16 or a multiple of 16) */
};


/* Optional knobs; pass NULL for all defaults. Zero means "automatic". */
typedef struct fd_options {
    int force_num_splits; /* > 0: about this many splits of the longest sequence (chunk = the largest
                             multiple of FD_CHUNK_QUANTUM not above max_len / n, at least the quantum) */
    int force_chunk;      /* > 0: the split stride, a multiple of FD_CHUNK_QUANTUM (wins over force_num_splits) */
    int force_kernel;     /* FD_KERNEL_* */
    int debug_checks;     /* 0 or 1. Paged calls with 1: the split kernels check every block-table
                             entry they address ([0, num_pages)) and every sequence length
                             ([0, min(max_seq_len, max_blocks * page_size)]) and record the first
                             violation in the workspace (fd_plan.ws_err_offset). They still clamp,
                             so no access leaves the cache. The call then waits for its kernels
                             (it synchronises `stream`; not for graph capture) and returns
                             FD_ERR_BAD_DATA, naming the sequence, table index and value, if any
                             check failed. Contiguous calls have no device-side index to check and
                             ignore it. The tables the pages' paged kernel reads are padded with -1
                             past each sequence's pages ("FlashAttention 与推理算子", section
                             "一个分页 decode attention kernel（支持 GQA）"): entries past
                             ceil(L_b / page_size) are never read and never reported. */
    void *split_begin_event; /* hipEvent_t stamped when the split kernel starts executing, or NULL */
    void *split_end_event;   /* hipEvent_t stamped when the split kernel finishes, or NULL
                                (both set by the dispatch itself: hipExtLaunchKernel) */
    int force_merge;         /* FD_MERGE_*: how the partials of a multi-split plan are merged;
                                FD_MERGE_FUSED is for contiguous caches (at most 32 splits and 64
                                (head, split) rows per workgroup), elsewhere FD_ERR_UNSUPPORTED */
    int force_launch;        /* FD_LAUNCH_*: paged calls only (contiguous ones launch a grid);
                                FD_LAUNCH_PERSISTENT needs B <= 1024, else FD_ERR_UNSUPPORTED */
} fd_options;

/* What a call with the same arguments would launch. */
typedef struct fd_plan {
    int kernel;          /* FD_KERNEL_VALU or FD_KERNEL_MFMA */
    int heads_per_group; /* query heads of one KV head that one workgroup computes (they share its rows) */
    int chunk;           /* split stride: every split but a sequence's last holds this many tokens */
    int num_splits;      /* splits of the longest sequence = grid y: ceil(max_len / chunk) for a paged
                            batch, max(1, floor(S / chunk)) for a contiguous cache (at least 1) */
    int grid_x, grid_y, grid_z; /* split kernel grid: (head_slices, splits, sequences); see work_list
                                   and persistent */
    int threads;         /* split kernel workgroup size */
    int merge;           /* 0: one split per sequence, o written directly; 1 (FD_MERGE_KERNEL): partials
                            go to the workspace and a merge kernel runs; 2 (FD_MERGE_FUSED, contiguous caches
                            only): one launch, the last workgroup of each head slice merges its partials */
    int kv_heads_per_group; /* adjacent KV heads one workgroup reads together (vector-ALU kernel with
                               H == Hkv: 2, or 4 for an E4M3 cache; else 1) */
    size_t workspace_bytes; /* bytes the workspace must hold (0 when merge == 0 and no debug record) */
    size_t ws_lse_offset;   /* byte offset of ws_lse inside the workspace */
    int work_list;          /* 1 (paged only): grid_y numbers the splits that hold tokens (the full
                               splits sequence by sequence, then the remainder splits largest first,
                               empty sequences last), grid_z = 1, one split per workgroup; chosen
                               when the (splits x sequences) grid would be mostly empty splits and
                               total_kv is known */
    int persistent;         /* 1 (paged only): grid_x = one workgroup per resident slot (two per compute
                               unit), grid_y = grid_z = 1; every workgroup numbers the items as the work
                               list does (units = items x head slices, largest first), starts with its
                               own unit (workgroup x takes unit x) and, each time a unit is done,
                               claims the next from a counter in the workspace's counter block until
                               none is left. Chosen when the units would take more than one round of
                               resident workgroups (B <= 1024). The split stride, the splits and so
                               the results are those of the grid form; total_kv only sizes the
                               splits (every item is processed). */
    size_t ws_err_offset;   /* paged plans with debug_checks: byte offset of the 16-byte error
                               record (int32 kind, sequence, table index or 0, offending value;
                               kind 1 = table entry, 2 = sequence length) inside the workspace,
                               which workspace_bytes then includes; 0 otherwise */
    size_t ws_o_offset;     /* byte offset of ws_o inside the workspace (FD_WS_COUNTER_BYTES) */
    int head_slices;        /* Hkv / kv_heads_per_group * (H / Hkv) / heads_per_group: workgroup-sized
                               slices of the heads of one sequence */
    int reserved3;
} fd_plan;

/*
 * Workspace layout when merge != 0 (every plan uses the same head block, so one
 * workspace serves calls of any plan):
 *   counters [FD_WS_COUNTER_BYTES / 4] uint32 at byte 0: a fused launch
 *                                (contiguous cache) counts the finished splits
 *                                of each head slice from the start of the
 *                                block, a persistent launch its claims and its
 *                                finished workgroups in the last 640 words
 *                                (10 counters, 256 bytes apart). They must be
 *                                ZERO before the workspace
 *                                is first used (e.g. hipMemset once after
 *                                allocating it); every completed call leaves
 *                                them zero. A persistent plan needs this block
 *                                even when it has one split (workspace_bytes
 *                                >= FD_WS_COUNTER_BYTES).
 *   ws_o  [B, H, num_splits, D]  fp32, normalised output of each split, at
 *                                byte offset ws_o_offset
 *   ws_lse[B, H, num_splits]     fp32, natural-log log-sum-exp of each split's
 *                                scores, at byte offset ws_lse_offset.
 * ws_o and ws_lse need no initialisation; the debug record, when asked for,
 * follows at ws_err_offset and is cleared by the call itself.
 * Split s < n_b - 1 of a sequence covers tokens [s*chunk, (s+1)*chunk) and the
 * last split runs to the sequence's end. A paged sequence of L_b tokens has
 * n_b = ceil(L_b / chunk) splits, the cut of "[CUDA 优化实战] 纯手搓 flash decoding
 * sm120", section "1. flash decoding": the last one holds the remainder (1 ..
 * chunk tokens); a batch's short remainder splits are scheduled last, largest
 * first, and fill the end of the launch. A contiguous cache of S tokens (one
 * sequence, every split in one round of workgroups) has max(1, floor(S /
 * chunk)) splits, the last one also taking the remainder (chunk .. 2*chunk - 1
 * tokens), so no short split straggles. Either way L = 0 has no split. Only
 * the splits of sequences with n_b > 1 are written; a sequence with one split
 * is written to o directly (and in a fused launch the last split's workgroup
 * merges). The split kernel stores partials as "[CUDA 优化实战] 纯手搓 flash
 * decoding sm120", section "2. kernel 实现细节" describes: normalised output plus
 * log-sum-exp.
 */

/* Compute units of the current HIP device (cached per device); -1 on error. */
int fd_device_num_cus(void);

/*
 * Plan of fd_decode. num_cus > 0 uses that compute-unit count (pure host
 * arithmetic, no GPU needed); num_cus == 0 queries the current device.
 * Argument meaning as in fd_decode.
 */
fd_status fd_decode_plan(int H, int Hkv, int S, int D, fd_dtype dtype, int num_cus,
                         const fd_options *opt, fd_plan *out);

/* Plan of fd_paged_decode; arguments as there. */
fd_status fd_paged_plan(int B, int H, int Hkv, int D, fd_dtype dtype, int page_size,
                        int max_seq_len, long long total_kv, int num_cus,
                        const fd_options *opt, fd_plan *out);

/*
 * Workspace bytes a call with these arguments needs (fd_plan.workspace_bytes of
 * the matching plan; 0 when every sequence fits one split and no debug record is
 * asked for). The split planner of "[CUDA 优化实战] 纯手搓 flash decoding sm120",
 * section "1. flash decoding" sizes the per-split output and log-sum-exp buffers
 * the same way: one row of D + 1 floats per (sequence, head, split). num_cus as
 * in the plan calls. *bytes is written only on FD_OK.
 */
fd_status fd_decode_workspace_size(int H, int Hkv, int S, int D, fd_dtype dtype, int num_cus,
                                   const fd_options *opt, size_t *bytes);
fd_status fd_paged_workspace_size(int B, int H, int Hkv, int D, fd_dtype dtype, int page_size,
                                  int max_seq_len, long long total_kv, int num_cus,
                                  const fd_options *opt, size_t *bytes);

/*
 * Single decode over a contiguous KV cache ("[CUDA 优化实战] 纯手搓 flash
 * decoding sm120", section "1. flash decoding": q [head, dim], kv [seq, head,
 * dim]).
 *   q  [H, D]          query, one row per head
 *   k  [S, Hkv, D]     keys, token-major
 *   v  [S, Hkv, D]     values, token-major
 *   o  [H, D]          output, fully overwritten (S == 0 gives zeros)
 *   scale              softmax scale (callers usually pass 1/sqrt(D)); any finite value,
 *                      negative and zero included, whose product with log2(e) (and
 *                      k_scale, for an FP8 cache) is finite, else FD_ERR_INVALID_ARG
 *   ws, ws_bytes       caller-owned device workspace of at least
 *                      fd_plan.workspace_bytes (may be NULL when that is 0)
 *   opt                NULL or options; stream: hipStream_t or NULL.
 */
fd_status fd_decode(const void *q, const void *k, const void *v, void *o,
                    int H, int Hkv, int S, int D, fd_dtype dtype, float scale,
                    void *ws, size_t ws_bytes, const fd_options *opt, void *stream);

/*
 * Batched decode over a paged KV cache with grouped-query heads
 * ("FlashAttention 与推理算子", sections "PagedAttention" and "一个分页 decode
 * attention kernel（支持 GQA）": token t of sequence b is slot t % page_size of
 * physical page block_table[b][t / page_size]).
 *   q            [B, H, D]
 *   k_cache      [num_pages, page_size, Hkv, D]
 *   v_cache      [num_pages, page_size, Hkv, D]
 *   block_table  [B, max_blocks] int32, device; entries past ceil(L_b/page_size)
 *                are never read (padding such as -1 is fine). Entries that are
 *                read must lie in [0, num_pages); others are clamped into that
 *                range (that sequence's output is then unspecified, but no
 *                access leaves the cache), and fd_options.debug_checks turns
 *                them into FD_ERR_BAD_DATA.
 *   seq_lens     [B] int32, device; L_b, clamped to [0, min(max_seq_len,
 *                max_blocks * page_size)]; L_b == 0 gives o[b] = 0.
 *   page_size    tokens per page, a power of two in [1, 1024]
 *   o            [B, H, D], fully overwritten
 *   max_seq_len  host-side upper bound of every L_b (sizes the grid; no
 *                device-to-host read of seq_lens ever happens)
 *   total_kv     host-side sum of L_b (each clamped to max_seq_len and to the
 *                table's reach) if known (> 0), else <= 0. It sizes the splits
 *                and, for a batch far shorter than its longest sequence, the
 *                work-list grid (fd_plan.work_list); in a work-list grid a value
 *                below the true sum leaves splits unlaunched, whose outputs are
 *                then NaN (a persistent launch processes every split whatever
 *                the value). A larger value only costs idle workgroups.
 *   Other arguments as in fd_decode.
 */
fd_status fd_paged_decode(const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *block_table, const int32_t *seq_lens, int page_size,
                          void *o, float scale, int B, int H, int Hkv, int D, int num_pages,
                          int max_blocks, int max_seq_len, long long total_kv, fd_dtype dtype,
                          void *ws, size_t ws_bytes, const fd_options *opt, void *stream);

/*
 * fd_paged_decode without a caller workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc. Arguments, plan and results are those of
 * fd_paged_decode without ws / ws_bytes. Nothing is allocated, by the call or
 * by any routine it calls: the partials (and counters, and the debug record)
 * live in a static device array of FD_NOALLOC_SCRATCH_BYTES (64 MiB) that the
 * library holds on every GPU it runs on until the process ends.
 *   - A call whose plan needs more (fd_plan.workspace_bytes of fd_paged_plan)
 *     returns FD_ERR_WORKSPACE before launching anything; a larger
 *     fd_options.force_chunk (fewer splits) shrinks the need.
 *   - Every call on a GPU shares that GPU's array, which keeps the last call's
 *     contents. Calls that overlap on one GPU (different streams or threads)
 *     RACE on it: the caller must order them.
 *   - The first call on a device also launches a small fill kernel on `stream`
 *     that zeroes the counter block at the head of the array.
 * Errors as for fd_paged_decode.
 */
fd_status fd_paged_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *block_table, const int32_t *seq_lens, int page_size, void *o,
                                  float scale, int B, int H, int Hkv, int D, int num_pages, int max_blocks,
                                  int max_seq_len, long long total_kv, fd_dtype dtype, const fd_options *opt,
                                  void *stream);

/*
 * FP8 KV cache. "FlashAttention 与推理算子", in the improvements listed after its
 * paged GQA kernel, notes that a real KV cache is BF16 or FP8, read with
 * 128-bit loads and converted to FP32 in registers. Here every K and V element
 * is an OCP FP8 E4M3 code (bias 7, 3 mantissa bits, no infinities, max 448)
 * and the cached value is code x k_scale (K) or code x v_scale (V).
 * Arguments as in fd_decode / fd_paged_decode, except:
 *   k, v / k_cache, v_cache   E4M3 codes, same shapes, 1 byte per element
 *                             (16-byte aligned as before)
 *   dtype                     FD_DTYPE_F16_KV_E4M3 or FD_DTYPE_BF16_KV_E4M3:
 *                             q and o are f16 / bf16
 *   k_scale, v_scale          finite dequantisation scales of K and V
 * The codes are converted exactly (to fp32 or, on the matrix cores, to the
 * query type) and accumulated in fp32.
 */
fd_status fd_decode_fp8kv(const void *q, const void *k, const void *v, void *o,
                          int H, int Hkv, int S, int D, fd_dtype dtype, float scale,
                          float k_scale, float v_scale,
                          void *ws, size_t ws_bytes, const fd_options *opt, void *stream);

fd_status fd_paged_decode_fp8kv(const void *q, const void *k_cache, const void *v_cache,
                                const int32_t *block_table, const int32_t *seq_lens, int page_size,
                                void *o, float scale, float k_scale, float v_scale,
                                int B, int H, int Hkv, int D, int num_pages,
                                int max_blocks, int max_seq_len, long long total_kv, fd_dtype dtype,
                                void *ws, size_t ws_bytes, const fd_options *opt, void *stream);

/*
 * Prefill attention: many queries over a prompt, optionally causal
 * ("FlashAttention 与推理算子", sections "标准注意力的问题" and
 * "FlashAttention：分块 + online softmax", its paragraph on the causal mask of
 * decoder self-attention). For every sequence b, position i < N and head h:
 *
 *     o[b,i,h,:] = sum_j softmax_j(scale * q[b,i,h,:] . k[b,j,g,:]) * v[b,j,g,:]
 *
 * over keys j < N, or j <= i when causal != 0; g = h / (H / Hkv).
 *   q, o   [B, N, H, D] row-major; o fully overwritten
 *   k, v   [B, N, Hkv, D] row-major (per sequence the decode cache layout)
 *   dtype  FD_DTYPE_F16 or FD_DTYPE_BF16 (matrix cores); D = 128
 *   N      0 .. 2^30 (N = 0 launches nothing); B, H <= 65535 and
 *          B * H * ceil(N / 64) < 2^31 (else FD_ERR_UNSUPPORTED)
 *   scale  any finite value (a negative one flips the sign of every score)
 *   ws, ws_bytes  bf16 only (f16 ignores them), device memory that must not
 *          overlap q, k, v or o. NULL: P.V runs on bf16 MFMAs with P split
 *          into two bf16 parts (two MFMAs per step). Otherwise at least
 *          fd_prefill_workspace_size() bytes (else FD_ERR_WORKSPACE), 16-byte
 *          aligned: a first kernel writes an f16 copy of V there (exact for
 *          |v| < 65536) and a flag per chunk of each sequence's V, the
 *          attention then runs P.V on f16 MFMAs with P in f16 (one MFMA per
 *          step), and a last kernel reruns, with the split P, the sequences
 *          whose V held a finite value of 65536 or more. Results agree
 *          within the same tolerance either way.
 *   opt    may be NULL; only split_begin_event / split_end_event are used, and
 *          they time the kernel that runs the attention of the sequences
 *          (with a workspace: the f16-V kernel alone)
 * Asynchronous on `stream`; errors as for fd_decode. The workspace is
 * read and written on `stream`: calls that share one may not overlap.
 */
fd_status fd_prefill(const void *q, const void *k, const void *v, void *o, int B, int N, int H, int Hkv, int D,
                     fd_dtype dtype, float scale, int causal, void *ws, size_t ws_bytes, const fd_options *opt,
                     void *stream);

/*
 * Workspace bytes fd_prefill uses for a bf16 prefill of these sizes: the f16
 * copy of V (B * N * Hkv * D * 2 bytes) and 1024 flag bytes per sequence.
 * 0 for f16, for arguments fd_prefill would refuse, and for N = 0.
 */
size_t fd_prefill_workspace_size(int B, int N, int Hkv, int D, fd_dtype dtype);

/* Static name of a status code. */
const char *fd_status_string(fd_status s);

/* Message of the last failing call on this thread ("" if none). */
const char *fd_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FD_H_ */

// fd_merge.hip -- log-sum-exp merge of the split partials (gfx950, wave64).
//
// One wave per (sequence b, query head h). Split s holds a normalised output
// O_s and the natural-log log-sum-exp lse_s of its scores. With
// M = max_s lse_s, w_s = exp(lse_s - M):  o = sum_s w_s O_s / sum_s w_s, which
// is the merge of "[CUDA 优化实战] 纯手搓 flash decoding sm120", section "2. kernel
// 实现细节" (weights exp(lse_s - global lse)) and equals the (m, l) form of
// "FlashAttention 与推理算子", section "decode 阶段的并行：Flash-Decoding 与
// split-K", since lse_s = m_s + ln l_s. Only the ceil(L_b / chunk) splits that
// hold tokens are read; a sequence with no token gets o = 0. Each lane owns two
// adjacent output elements, so a split's 512-byte partial row is one coalesced
// 8-byte-per-lane load. Sequences that fit one split were written directly by
// the split kernel and are skipped here.
#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

template <typename T, bool PAGED>
__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    int L = a.max_len;
    if (PAGED) L = max(0, min(a.seq_lens[b], a.max_len));
    const int n = min((L + a.chunk - 1) / a.chunk, a.num_splits);
    if (n == 1) return;  // the split kernel wrote this row directly
    const size_t bh = (size_t)b * a.H + h;
    const float2 o = merge_partials(a.ws_o + bh * a.num_splits * kHeadDim, a.ws_lse + bh * a.num_splits, n, lane);
    store_out_pair<T>(a.out, bh, lane, o);
}

template <typename T, bool PAGED>
hipError_t launch_one(int B, const MergeArgs &a, hipStream_t st) {
    MergeArgs arg = a;
    void *args[] = {&arg};
    return hipLaunchKernel(reinterpret_cast<const void *>(&merge_kernel<T, PAGED>), dim3(a.H, B), dim3(64), args, 0,
                           st);
}

}  // namespace

hipError_t launch_merge(fd_dtype dtype, bool paged, int B, const MergeArgs &a, hipStream_t st) {
    switch (dtype) {
        case FD_DTYPE_F32: return paged ? launch_one<float, true>(B, a, st) : launch_one<float, false>(B, a, st);
        case FD_DTYPE_F16: return paged ? launch_one<_Float16, true>(B, a, st) : launch_one<_Float16, false>(B, a, st);
        case FD_DTYPE_BF16: return paged ? launch_one<__bf16, true>(B, a, st) : launch_one<__bf16, false>(B, a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace fd

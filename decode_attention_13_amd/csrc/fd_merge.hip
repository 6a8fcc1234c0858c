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
// 8-byte-per-lane load.
#include "fd_device.h"
#include "fd_internal.h"

namespace fd {

namespace {

template <typename T>
struct Pair;
template <>
struct Pair<float> {
    typedef float2 type;
    __device__ static type make(float a, float b) { return make_float2(a, b); }
};
template <>
struct Pair<__bf16> {
    typedef __bf16 type __attribute__((ext_vector_type(2)));
    __device__ static type make(float a, float b) { return type{(__bf16)a, (__bf16)b}; }
};
template <>
struct Pair<_Float16> {
    typedef _Float16 type __attribute__((ext_vector_type(2)));
    __device__ static type make(float a, float b) { return type{(_Float16)a, (_Float16)b}; }
};

template <typename T, bool PAGED>
__global__ __launch_bounds__(64) void merge_kernel(MergeArgs a) {
    const int h = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    int L = a.max_len;
    if (PAGED) L = max(0, min(a.seq_lens[b], a.max_len));
    const int n = min((L + a.chunk - 1) / a.chunk, a.num_splits);
    const size_t row0 = ((size_t)b * a.H + h) * a.num_splits;
    const float *lse = a.ws_lse + row0;

    float mx = -INFINITY;
    for (int s = lane; s < n; s += 64) mx = fmaxf(mx, lse[s]);
    mx = wave_max(mx);
    const float mu = finite_or_zero(mx);

    // Splits in groups of 64: lane i computes split (s0 + i)'s weight, the
    // weights reach every lane through readlane, and each lane accumulates its
    // two output elements with 8 independent loads in flight.
    const float2 *src = reinterpret_cast<const float2 *>(a.ws_o + row0 * kHeadDim) + lane;
    float o0 = 0.f, o1 = 0.f, wpart = 0.f;
    for (int s0 = 0; s0 < n; s0 += 64) {
        const int cnt = min(64, n - s0);
        const float w = lane < cnt ? exp2_fast((lse[s0 + lane] - mu) * kLog2e) : 0.f;
        wpart += w;
        for (int i = 0; i < cnt; i += 8) {
            float2 x[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (i + u < cnt) x[u] = src[(size_t)(s0 + i + u) * (kHeadDim / 2)];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (i + u < cnt) {
                    const float wu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), i + u));
                    o0 = __builtin_fmaf(wu, x[u].x, o0);
                    o1 = __builtin_fmaf(wu, x[u].y, o1);
                }
            }
        }
    }
    const float wsum = wave_sum(wpart);
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    typedef typename Pair<T>::type P2;
    P2 *out = reinterpret_cast<P2 *>(reinterpret_cast<T *>(a.out) + ((size_t)b * a.H + h) * kHeadDim) + lane;
    *out = Pair<T>::make(o0 * inv, o1 * inv);
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

// Plan of a packed variable-length prefill (gfx950): from the caller's sequence boundaries
// to the table every prefill kernel reads (VarlenPlan in gdr_launch.h).  The pages route
// work by sequence length (ExecuTorch PR #21021, second commit summary) but give no batch
// format; sequences laid end to end with their boundaries in an array is the plainest one.
//
// One workgroup of 1024 threads: sanitised starts (clamped to [0, T], running maximum),
// chunk counts ceil(len / C) and their exclusive prefix (each by a blocked scan over the
// threads), then the sequence of every chunk slot by a binary search over the prefix in LDS.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {
namespace {

constexpr int kPlanThreads = 1024;

// Inclusive scan of one value per thread over the workgroup (max or sum), in place in `part`.
template <bool MAX>
__device__ __forceinline__ int block_scan(int* part, int x) {
    const int tid = threadIdx.x;
    part[tid] = x;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int y = tid >= off ? part[tid - off] : 0;
        __syncthreads();
        part[tid] = MAX ? max(part[tid], y) : part[tid] + y;
        __syncthreads();
    }
    return part[tid];
}

__global__ __launch_bounds__(kPlanThreads) void varlen_plan_kernel(const int32_t* __restrict__ cu, int B, int T,
                                                                   int C, int nct, int32_t* __restrict__ plan) {
    __shared__ int sStart[kVarlenMaxSeqs + 1];
    __shared__ int sFirst[kVarlenMaxSeqs + 1];
    __shared__ int sPart[kPlanThreads];
    const int tid = threadIdx.x;

    // 1. starts: each thread a run of the B + 1 entries, clamped and made non-decreasing
    const int per = (B + 1 + kPlanThreads - 1) / kPlanThreads;
    const int e0 = min(tid * per, B + 1), e1 = min(e0 + per, B + 1);
    int m = 0;
    for (int e = e0; e < e1; ++e) {
        m = max(m, min(max(cu[e], 0), T));
        sStart[e] = m;
    }
    block_scan<true>(sPart, m);
    const int before = tid > 0 ? sPart[tid - 1] : 0;
    for (int e = e0; e < e1; ++e) sStart[e] = max(sStart[e], before);
    __syncthreads();

    // 2. chunks per sequence and their exclusive prefix
    const int ps = (B + kPlanThreads - 1) / kPlanThreads;
    const int i0 = min(tid * ps, B), i1 = min(i0 + ps, B);
    int sum = 0;
    for (int i = i0; i < i1; ++i) sum += (sStart[i + 1] - sStart[i] + C - 1) / C;
    block_scan<false>(sPart, sum);
    int acc = tid > 0 ? sPart[tid - 1] : 0;
    for (int i = i0; i < i1; ++i) {
        sFirst[i] = acc;
        acc += (sStart[i + 1] - sStart[i] + C - 1) / C;
    }
    if (tid == kPlanThreads - 1) sFirst[B] = sPart[kPlanThreads - 1];
    __syncthreads();

    for (int e = tid; e <= B; e += kPlanThreads) {
        plan[VarlenPlan::starts(B) + e] = sStart[e];
        plan[VarlenPlan::first(B) + e] = sFirst[e];
    }
    // 3. sequence of each chunk slot: the last sequence whose first slot is <= the slot (a
    //    sequence without rows shares its first slot with the next one)
    const int total = min(sFirst[B], nct);
    for (int c = tid; c < total; c += kPlanThreads) {
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sFirst[mid] <= c) lo = mid;
            else hi = mid - 1;
        }
        plan[VarlenPlan::chunk_seq(B) + c] = lo;
    }
}

}  // namespace

hipError_t launch_varlen_plan(const LaunchArgs& a) {
    if (a.B < 1 || a.B > kVarlenMaxSeqs || !a.cu_seqlens || !a.plan) return hipErrorInvalidValue;
    hipLaunchKernelGGL(varlen_plan_kernel, dim3(1), dim3(kPlanThreads), 0, (hipStream_t)a.stream, a.cu_seqlens,
                       a.B, a.T, a.chunk, a.nct, a.plan);
    return hipGetLastError();
}

}  // namespace gdr

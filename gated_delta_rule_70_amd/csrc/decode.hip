// Decode step of the channelwise gated delta rule (T == 1), gfx950.
//
// The two-pass token recurrence of ExecuTorch PR #21021 ("Reorder channelwise gated delta
// rule chunked hot loops for autovectorization", first commit summary), mapped to a
// memory-bound GPU kernel:
//   pass 1: pred_j = sum_i exp(g_i) S_ij k_i              (decay folded into the prediction)
//   pass 2: S_ij  <- exp(g_i) S_ij + k_i beta (v_j - pred_j);   o_j = sum_i S_ij q_i
// The state slice a workgroup owns is loaded from HBM once into registers, kept there
// between the passes and stored once: one read and one write of S per step, the minimum.
//
// Launch: one 256-thread workgroup per (batch, value head, BVD-wide column block).
// Thread t owns column quad cq = t % (BVD/4) (a float4 of columns) and the rows
// rl, rl + NRL, ... with rl = t / (BVD/4); a wave therefore touches 64/(BVD/4) rows with
// fully coalesced 16-byte loads along dv.  Column sums over rows are reduced first with
// cross-lane shuffles inside the wave, then across the four waves through LDS.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

template <typename TIn, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(const TIn* __restrict__ q,
                                                     const TIn* __restrict__ k,
                                                     const TIn* __restrict__ v,
                                                     const float* __restrict__ g,
                                                     const float* __restrict__ beta,
                                                     const float* h0, float* __restrict__ o,
                                                     float* ht, int HK, int HV) {
    constexpr int BVD = DV < 64 ? DV : 64;   // columns per workgroup
    constexpr int NQ = BVD / 4;              // column quads per row
    constexpr int NRL = 256 / NQ;            // row lanes
    constexpr int RPT = DK / NRL;            // rows per thread
    constexpr int LPW = 64 / NQ;             // row lanes per wave
    static_assert(RPT >= 1 && DK % NRL == 0, "unsupported dk/dv combination");

    __shared__ f32x4 red[4][NQ];

    const int ncb = DV / BVD;
    const int blk = blockIdx.x;
    const int cb = blk % ncb;
    const int bh = blk / ncb;  // b * HV + h
    const int h = bh % HV;
    const int b = bh / HV;
    const int kh = h / (HV / HK);
    const int t = threadIdx.x;
    const int cq = t % NQ;
    const int rl = t / NQ;
    const int wave = t >> 6;
    const int col = cb * BVD + 4 * cq;

    const size_t sbase = (size_t)bh * DK * DV + col;
    f32x4 S[RPT];
    if (h0 != nullptr) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            S[m] = *reinterpret_cast<const f32x4*>(h0 + sbase + (size_t)(rl + NRL * m) * DV);
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const size_t kq = ((size_t)b * HK + kh) * DK;
    const size_t gb = (size_t)bh * DK;
    float e[RPT], kk[RPT], qq[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rl + NRL * m;
        e[m] = __expf(g[gb + i]);
        kk[m] = to_f32(k[kq + i]);
        qq[m] = to_f32(q[kq + i]);
    }

    // pass 1: prediction with the decay folded in
    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        S[m] *= e[m];
        p += S[m] * kk[m];
    }
#pragma unroll
    for (int off = NQ; off < 64; off <<= 1) {
        p.x += __shfl_xor(p.x, off);
        p.y += __shfl_xor(p.y, off);
        p.z += __shfl_xor(p.z, off);
        p.w += __shfl_xor(p.w, off);
    }
    if ((t & 63) < NQ) red[wave][cq] = p;
    __syncthreads();
    const f32x4 pred = red[0][cq] + red[1][cq] + red[2][cq] + red[3][cq];

    const float bt = beta[bh];
    const size_t vb = (size_t)bh * DV + col;
    const f32x4 vv = {to_f32(v[vb + 0]), to_f32(v[vb + 1]), to_f32(v[vb + 2]), to_f32(v[vb + 3])};
    const f32x4 d = (vv - pred) * bt;

    // pass 2: rank-one update of the (already decayed) state, output partial sums
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        S[m] += d * kk[m];
        acc += S[m] * qq[m];
    }
    if (ht != nullptr) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            *reinterpret_cast<f32x4*>(ht + sbase + (size_t)(rl + NRL * m) * DV) = S[m];
    }
#pragma unroll
    for (int off = NQ; off < 64; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off);
        acc.y += __shfl_xor(acc.y, off);
        acc.z += __shfl_xor(acc.z, off);
        acc.w += __shfl_xor(acc.w, off);
    }
    __syncthreads();  // every wave has read red[] for pred
    if ((t & 63) < NQ) red[wave][cq] = acc;
    __syncthreads();
    if (t < NQ) {
        const f32x4 out = red[0][cq] + red[1][cq] + red[2][cq] + red[3][cq];
        *reinterpret_cast<f32x4*>(o + vb) = out;
    }
    (void)LPW;
}

template <typename TIn, int DK, int DV>
static hipError_t launch_decode_t(const LaunchArgs& a) {
    constexpr int BVD = DV < 64 ? DV : 64;
    const long long nblk = (long long)a.B * a.HV * (DV / BVD);
    hipLaunchKernelGGL((decode_kernel<TIn, DK, DV>), dim3((unsigned)nblk), dim3(256), 0,
                       (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v,
                       a.g, a.beta, a.h0, a.o, a.ht, a.HK, a.HV);
    return hipGetLastError();
}

template <typename TIn>
static hipError_t dispatch_dims(const LaunchArgs& a) {
#define GDR_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_decode_t<TIn, DK_, DV_>(a);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const LaunchArgs& a) {
    return a.qkv_f32 ? dispatch_dims<float>(a) : dispatch_dims<bf16_t>(a);
}

}  // namespace gdr

// Token recurrence of the channelwise gated delta rule, gfx950: the decode step (T == 1)
// and the fused recurrent form for short multi-token calls (T tokens in one launch).
//
// The two-pass token recurrence of ExecuTorch PR #21021 ("Reorder channelwise gated delta
// rule chunked hot loops for autovectorization", first commit summary), mapped to a
// memory-bound GPU kernel; per token:
//   pass 1: pred_j = sum_i exp(g_i) S_ij k_i              (decay folded into the prediction)
//   pass 2: S_ij  <- exp(g_i) S_ij + k_i beta (v_j - pred_j);   o_j = sum_i S_ij q_i
// The state slice a workgroup owns is loaded from HBM once into registers, kept there
// across the passes and across all T tokens of the call, and stored once: one read and one
// write of S per call, the minimum.  The page routes only T == 1 to this path (commit
// summary 2 of the same PR); running it for T > 1 in one launch is what short calls
// (speculative chains, a few tokens) use instead of T separate decode steps.
//
// Launch: one 256-thread workgroup per (batch, value head, BVD-wide column block).
// Thread t owns column quad cq = t % (BVD/4) (a float4 of columns) and the rows
// rl, rl + NRL, ... with rl = t / (BVD/4); a wave therefore touches 64/(BVD/4) rows with
// fully coalesced 16-byte loads along dv.  Column sums over rows are reduced first with
// cross-lane shuffles inside the wave, then across the four waves through LDS (two
// barriers per token; the two reduction buffers alternate so no third one is needed).
// The next token's inputs are requested while the current one is processed.
//
// The state is loaded and stored with non-temporal hints: each element is touched once per
// call, and between decode steps of a real model the state of every other layer passes
// through the caches, so keeping it cached buys nothing.  Measured at B = 32, HV = 32,
// 128 x 128, steps cycling over 8 states (512 MiB, HBM-resident) replayed from a graph:
// 23.5 us per step (72 % of the 8 TB/s peak) against 29.1 us with ordinary accesses; a
// single state replayed in place (then held in the 256 MB last-level cache) goes from 20.8
// to 22.9 us.
//
// Fused input prologue (template flags KN, GS): with raw keys (KN) the prediction is formed
// with the raw key and scaled by 1 / |k|_2 after its reduction (it is linear in k), the
// sum of squares riding along in the same reduction, and the update uses d / |k|_2; with gate
// logits (GS) the decay factor is exp(-softplus(a)) = 1 / (1 + e^a).
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

template <typename TIn, typename TG, int DK, int DV, bool KN, bool GS>
__global__ __launch_bounds__(256) void token_kernel(const TIn* __restrict__ q,
                                                    const TIn* __restrict__ k,
                                                    const TIn* __restrict__ v,
                                                    const TG* __restrict__ g,
                                                    const float* __restrict__ beta,
                                                    const float* h0, void* __restrict__ o,
                                                    float* ht, int T, int HK, int HV, int HG,
                                                    const int32_t* __restrict__ cu, int obf) {
    constexpr int BVD = DV < 64 ? DV : 64;   // columns per workgroup
    constexpr int NQ = BVD / 4;              // column quads per row
    constexpr int NRL = 256 / NQ;            // row lanes
    constexpr int RPT = DK / NRL;            // rows per thread
    static_assert(RPT >= 1 && DK % NRL == 0, "unsupported dk/dv combination");

    __shared__ f32x4 red_p[4][NQ];  // pass-1 partial sums of each wave
    __shared__ f32x4 red_o[4][NQ];  // output partial sums of each wave
    __shared__ float red_k[4];      // each wave's sum of squared key entries (raw keys)

    const int ncb = DV / BVD;
    const int blk = blockIdx.x;
    const int cb = blk % ncb;
    const int bh = blk / ncb;  // b * HV + h
    const int h = bh % HV;
    const int b = bh / HV;
    const int kh = h / (HV / HK);
    const int tid = threadIdx.x;
    const int cq = tid % NQ;
    const int rl = tid / NQ;
    const int wave = tid >> 6;
    const int col = cb * BVD + 4 * cq;

    const size_t sbase = (size_t)bh * DK * DV + col;
    f32x4 S[RPT];
    if (h0 != nullptr) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            S[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(h0 + sbase + (size_t)(rl + NRL * m) * DV));
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Rows of this batch element, or of packed sequence b (cu != nullptr: rows
    // [cu[b], cu[b + 1]), both clamped to [0, T] so that no access leaves the tensors).
    size_t row0 = (size_t)b * T;
    int nt = T;
    if (cu != nullptr) {
        const int r0 = min(max(cu[b], 0), T);
        const int r1 = min(max(cu[b + 1], r0), T);
        row0 = (size_t)r0;
        nt = r1 - r0;
    }
    // Token tok of this (batch, head): q/k row, g row, v/o columns, beta.
    const size_t kq0 = (row0 * HK + kh) * DK;
    const size_t gb0 = (row0 * HG + h / (HV / HG)) * DK;  // gate head of h
    const size_t vb0 = (row0 * HV + h) * DV + col;
    const size_t bb0 = row0 * HV + h;
    const size_t kq_t = (size_t)HK * DK, gb_t = (size_t)HG * DK, vb_t = (size_t)HV * DV;

    // raw inputs of the next token, requested one token ahead
    float gn[RPT];
    TIn kn[RPT], qn[RPT], vn[4];
    float btn;
    auto request = [&](int tok) {
        const size_t kq = kq0 + tok * kq_t, gb = gb0 + tok * gb_t, vb = vb0 + tok * vb_t;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int i = rl + NRL * m;
            gn[m] = to_f32(g[gb + i]);
            kn[m] = k[kq + i];
            qn[m] = q[kq + i];
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) vn[c] = v[vb + c];
        btn = beta[bb0 + tok * HV];
    };
    if (nt > 0) request(0);

    for (int tok = 0; tok < nt; ++tok) {
        float e[RPT], kk[RPT], qq[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            e[m] = GS ? decay_from_logit(gn[m]) : __expf(gn[m]);
            kk[m] = to_f32(kn[m]);
            qq[m] = to_f32(qn[m]);
        }
        const f32x4 vv = {to_f32(vn[0]), to_f32(vn[1]), to_f32(vn[2]), to_f32(vn[3])};
        const float bt = btn;
        if (tok + 1 < nt) request(tok + 1);

        // pass 1: prediction with the decay folded in
        f32x4 p = {0.f, 0.f, 0.f, 0.f};
        float s2 = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            S[m] *= e[m];
            p += S[m] * kk[m];
            if constexpr (KN) s2 = fmaf(kk[m], kk[m], s2);
        }
#pragma unroll
        for (int off = NQ; off < 64; off <<= 1) {
            p.x += __shfl_xor(p.x, off);
            p.y += __shfl_xor(p.y, off);
            p.z += __shfl_xor(p.z, off);
            p.w += __shfl_xor(p.w, off);
            if constexpr (KN) s2 += __shfl_xor(s2, off);
        }
        // red_p is free: every thread read the previous token's sums before the previous
        // token's second barrier (likewise red_k)
        if ((tid & 63) < NQ) red_p[wave][cq] = p;
        if (KN && (tid & 63) == 0) red_k[wave] = s2;
        __syncthreads();
        f32x4 pred = red_p[0][cq] + red_p[1][cq] + red_p[2][cq] + red_p[3][cq];
        float rn = 1.f;
        if constexpr (KN) {
            rn = inv_key_norm(red_k[0] + red_k[1] + red_k[2] + red_k[3]);
            pred *= rn;
        }
        const f32x4 d = (vv - pred) * (bt * rn);  // d / |k|: the update then uses the raw key

        // pass 2: rank-one update of the (already decayed) state, output partial sums
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            S[m] += d * kk[m];
            acc += S[m] * qq[m];
        }
#pragma unroll
        for (int off = NQ; off < 64; off <<= 1) {
            acc.x += __shfl_xor(acc.x, off);
            acc.y += __shfl_xor(acc.y, off);
            acc.z += __shfl_xor(acc.z, off);
            acc.w += __shfl_xor(acc.w, off);
        }
        // red_o is free: its readers read the previous token's sums before this token's
        // first barrier
        if ((tid & 63) < NQ) red_o[wave][cq] = acc;
        __syncthreads();
        if (tid < NQ) {
            const f32x4 out = red_o[0][cq] + red_o[1][cq] + red_o[2][cq] + red_o[3][cq];
            store_o4(o, vb0 + tok * vb_t, out, obf);
        }
    }
    if (ht != nullptr) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            __builtin_nontemporal_store(S[m], reinterpret_cast<f32x4*>(ht + sbase + (size_t)(rl + NRL * m) * DV));
    }
}

// The decode step alone (T == 1): the same workgroup shape, thread-to-state mapping and
// operation order as token_kernel, so its results equal token_kernel's bit for bit, but
// without the next-token request buffers: the step's decay factors, keys and queries are
// staged once per workgroup in LDS (one load per thread instead of one per owned row).
// That keeps a thread within 64 registers, so eight waves fit per SIMD and every
// workgroup of a decode step is resident at once: the whole state is requested in one
// round instead of two.
template <typename TIn, typename TG, int DK, int DV, bool KN, bool GS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8, 8)))
void decode_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v,
                   const TG* __restrict__ g, const float* __restrict__ beta, const float* h0,
                   void* __restrict__ o, float* ht, int HK, int HV, int HG, int obf) {
    constexpr int BVD = DV < 64 ? DV : 64;
    constexpr int NQ = BVD / 4;
    constexpr int NRL = 256 / NQ;
    constexpr int RPT = DK / NRL;
    static_assert(RPT >= 1 && DK % NRL == 0 && DK <= 256, "unsupported dk/dv combination");

    __shared__ float s_e[DK], s_k[DK], s_q[DK];
    __shared__ f32x4 red_p[4][NQ];
    __shared__ f32x4 red_o[4][NQ];
    __shared__ float red_k[4];  // the key's sum of squares per staging wave (raw keys)

    const int ncb = DV / BVD;
    const int blk = blockIdx.x;
    const int cb = blk % ncb;
    const int bh = blk / ncb;
    const int h = bh % HV;
    const int b = bh / HV;
    const int kh = h / (HV / HK);
    const int tid = threadIdx.x;
    const int cq = tid % NQ;
    const int rl = tid / NQ;
    const int wave = tid >> 6;
    const int col = cb * BVD + 4 * cq;

    const size_t sbase = (size_t)bh * DK * DV + col;
    f32x4 S[RPT];
    if (h0 != nullptr) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            S[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(h0 + sbase + (size_t)(rl + NRL * m) * DV));
    } else {
#pragma unroll
        for (int m = 0; m < RPT; ++m) S[m] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const size_t kq = ((size_t)b * HK + kh) * DK;
    const size_t gb = ((size_t)b * HG + h / (HV / HG)) * DK;  // gate head of h
    const size_t vb = ((size_t)b * HV + h) * DV + col;
    if (tid < DK) {
        const float gv = to_f32(g[gb + tid]);
        s_e[tid] = GS ? decay_from_logit(gv) : __expf(gv);
        s_k[tid] = to_f32(k[kq + tid]);
        s_q[tid] = to_f32(q[kq + tid]);
    }
    if constexpr (KN) {  // the staging waves (threads < DK) reduce the key's sum of squares
        if (tid < ((DK + 63) & ~63)) {
            const float kx = tid < DK ? to_f32(k[kq + tid]) : 0.f;
            float s2 = kx * kx;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) s2 += __shfl_xor(s2, off);
            if ((tid & 63) == 0) red_k[wave] = s2;
        }
    }
    const f32x4 vv = {to_f32(v[vb]), to_f32(v[vb + 1]), to_f32(v[vb + 2]), to_f32(v[vb + 3])};
    const float bt = beta[(size_t)b * HV + h];
    __syncthreads();

    f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rl + NRL * m;
        S[m] *= s_e[i];
        p += S[m] * s_k[i];
    }
#pragma unroll
    for (int off = NQ; off < 64; off <<= 1) {
        p.x += __shfl_xor(p.x, off);
        p.y += __shfl_xor(p.y, off);
        p.z += __shfl_xor(p.z, off);
        p.w += __shfl_xor(p.w, off);
    }
    if ((tid & 63) < NQ) red_p[wave][cq] = p;
    __syncthreads();
    f32x4 pred = red_p[0][cq] + red_p[1][cq] + red_p[2][cq] + red_p[3][cq];
    float rn = 1.f;
    if constexpr (KN) {
        float s2 = red_k[0];
#pragma unroll
        for (int w2 = 1; w2 < (DK + 63) / 64; ++w2) s2 += red_k[w2];
        rn = inv_key_norm(s2);
        pred *= rn;  // the prediction with the normalised key
    }
    const f32x4 d = (vv - pred) * (bt * rn);  // d / |k|: the update then uses the raw key

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int i = rl + NRL * m;
        S[m] += d * s_k[i];
        acc += S[m] * s_q[i];
    }
#pragma unroll
    for (int off = NQ; off < 64; off <<= 1) {
        acc.x += __shfl_xor(acc.x, off);
        acc.y += __shfl_xor(acc.y, off);
        acc.z += __shfl_xor(acc.z, off);
        acc.w += __shfl_xor(acc.w, off);
    }
    if ((tid & 63) < NQ) red_o[wave][cq] = acc;
    __syncthreads();
    if (tid < NQ) {
        const f32x4 out = red_o[0][cq] + red_o[1][cq] + red_o[2][cq] + red_o[3][cq];
        store_o4(o, vb, out, obf);
    }
    if (ht != nullptr) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            __builtin_nontemporal_store(S[m], reinterpret_cast<f32x4*>(ht + sbase + (size_t)(rl + NRL * m) * DV));
    }
}

template <typename TIn, typename TG, int DK, int DV, bool KN, bool GS>
static hipError_t launch_tokens_t(const LaunchArgs& a) {
    constexpr int BVD = DV < 64 ? DV : 64;
    const long long nblk = (long long)a.B * a.HV * (DV / BVD);
    if (a.T == 1 && a.cu_seqlens == nullptr) {
        hipLaunchKernelGGL((decode_kernel<TIn, TG, DK, DV, KN, GS>), dim3((unsigned)nblk), dim3(256), 0,
                           (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v,
                           (const TG*)a.g, a.beta, a.h0, a.o, a.ht, a.HK, a.HV, a.HG, (int)a.o_bf16);
    } else {
        hipLaunchKernelGGL((token_kernel<TIn, TG, DK, DV, KN, GS>), dim3((unsigned)nblk), dim3(256), 0,
                           (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, (const TIn*)a.v,
                           (const TG*)a.g, a.beta, a.h0, a.o, a.ht, a.T, a.HK, a.HV, a.HG, a.cu_seqlens,
                           (int)a.o_bf16);
    }
    return hipGetLastError();
}

template <typename TIn, typename TG, bool KN, bool GS>
static hipError_t dispatch_dims(const LaunchArgs& a) {
#define GDR_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_tokens_t<TIn, TG, DK_, DV_, KN, GS>(a);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

// Decode step and fused recurrent call: decode_kernel for T == 1, token_kernel otherwise.
template <bool KN, bool GS>
static hipError_t dispatch_types(const LaunchArgs& a) {
    if (a.qkv_f32) return dispatch_dims<float, float, KN, GS>(a);
    return a.g_bf16 ? dispatch_dims<bf16_t, bf16_t, KN, GS>(a) : dispatch_dims<bf16_t, float, KN, GS>(a);
}

hipError_t launch_tokens(const LaunchArgs& a) {
    if (a.k_l2norm) return a.g_softplus ? dispatch_types<true, true>(a) : dispatch_types<true, false>(a);
    return a.g_softplus ? dispatch_types<false, true>(a) : dispatch_types<false, false>(a);
}

}  // namespace gdr

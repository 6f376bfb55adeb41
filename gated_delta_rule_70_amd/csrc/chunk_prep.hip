// Chunk-parallel half of the chunkwise WY/UT prefill (gfx950).
//
// ExecuTorch PR #21021 ("Reorder channelwise gated delta rule chunked hot loops for
// autovectorization", second commit summary) evaluates prefill chunk by chunk: per-channel
// log-decay prefixes, the beta-folded triangular transform, WY pseudo-keys and
// pseudo-values, causal query/key terms, then the inter-chunk state carry.  Everything
// except the carry depends on one chunk only, so this kernel runs it for all
// (batch, value head, chunk) triples at once -- one 256-thread workgroup each -- and hands
// the results to the sequential carry kernel as fp16 MFMA operand fragments.
//
// For a chunk of C tokens (rows r, s; gam = inclusive prefix of g inside the chunk):
//   gram     A_rs = beta_r sum_c k_rc k_sc exp(gam_rc - gam_sc)   (s < r)
//   causal   P_rs =        sum_c q_rc k_sc exp(gam_rc - gam_sc)   (s <= r)
//   solve    Tinv = (I + A)^-1 by exact 16x16-block forward substitution (the block TRSM
//            of uzu PR #576, "Support TreeUpdateSolve kernel", done in fp32 in LDS)
//   WY       Tb = Tinv diag(beta);  W = Tb (exp(gam) * K)           (pseudo-keys)
//   carry    Qt = exp(gam) * Q;  Kb = exp(gam_last - gam) * K;  exp(gam_last)
// Outputs per chunk (see ChunkRecord): Qt, -W, Kb^T, Tb, P as fragments, exp(gam_last).
//
// Decay factors inside the MFMA operands are split around a per-16-row-block reference
// row so no operand exceeds its format's range: for blocks J < I the reference is the
// last row of J, making both factors <= 1 (fp16 operands); for the diagonal blocks it is
// the block's 8th row, and operands are split into bf16 hi + lo parts (three products),
// which keeps ~16 significant bits with fp32's exponent range.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

template <typename TIn>
struct VecLoad;
template <>
struct VecLoad<float> {
    static constexpr int N = 4;
};
template <>
struct VecLoad<bf16_t> {
    static constexpr int N = 8;
};

template <typename TIn, int DK, int C>
__global__ __launch_bounds__(256) void chunk_prep_kernel(const TIn* __restrict__ q,
                                                         const TIn* __restrict__ k,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ beta,
                                                         unsigned char* __restrict__ ws, int T,
                                                         int HK, int HV, int NC) {
    constexpr int NB = C / 16;
    constexpr int NQS = (C + 31) / 32;
    constexpr int KC = DK / 32;
    constexpr int DKT = DK / 16;
    constexpr int GP = DK + 4;               // padded fp32 row (gam)
    constexpr int VN = VecLoad<TIn>::N;
    constexpr int XP = DK + VN;              // padded input row (k, q)
    constexpr int AP = C + 4;                // padded fp32 row (A, Tinv)
    constexpr int NSEG = 256 / DK;           // scan segments per channel
    constexpr int RPS = C / NSEG;            // rows per segment
    static_assert(RPS >= 1 && C % NSEG == 0, "chunk too short for this key dim");

    __shared__ float sGam[C * GP];
    __shared__ TIn sK[C * XP];
    __shared__ TIn sQ[C * XP];
    __shared__ float sA[C * AP];
    __shared__ float sT[C * AP];
    __shared__ float sBeta[C];
    __shared__ float sSeg[NSEG * DK];
    __shared__ float sY[(NB > 1 ? NB - 1 : 1) * 256];

    constexpr ChunkRecord R = ChunkRecord::make(C, DK);
    const int blk = blockIdx.x;
    const int n = blk % NC;
    const int bh = blk / NC;
    const int h = bh % HV;
    const int b = bh / HV;
    const int kh = h / (HV / HK);
    const int t0 = n * C;
    const int L = min(C, T - t0);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;
    const int gq = lane >> 4;

    unsigned char* rec = ws + (size_t)((size_t)bh * NC + n) * R.bytes;
    half8* frags = reinterpret_cast<half8*>(rec);
    float* egl_out = reinterpret_cast<float*>(rec + (size_t)R.nfrag * 1024);

    // ---- load g and form the inclusive per-channel prefix (two-level scan) -------------
    {
        const int c = tid % DK;
        const int seg = tid / DK;
        float loc[RPS];
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < RPS; ++m) {  // unconditional loads from clamped rows, then mask
            const int r = seg * RPS + m;
            const float gv = g[(((size_t)b * T + t0 + min(r, L - 1)) * HV + h) * DK + c];
            loc[m] = r < L ? gv : 0.f;
        }
#pragma unroll
        for (int m = 0; m < RPS; ++m) {
            acc += loc[m];
            loc[m] = acc;
        }
        sSeg[seg * DK + c] = acc;
        __syncthreads();
        float off = 0.f;
        for (int s2 = 0; s2 < seg; ++s2) off += sSeg[s2 * DK + c];
#pragma unroll
        for (int m = 0; m < RPS; ++m) sGam[(seg * RPS + m) * GP + c] = loc[m] + off;
    }
    // ---- load k, q rows (zero past the chunk end) and beta ------------------------------
    {
        constexpr int VPR = DK / VN;  // vectors per row
        for (int idx = tid; idx < C * VPR; idx += 256) {
            const int r = idx / VPR;
            const int cv = idx % VPR;
            const size_t off = (((size_t)b * T + t0 + min(r, L - 1)) * HK + kh) * DK + (size_t)cv * VN;
            uint4 kv = *reinterpret_cast<const uint4*>(k + off);
            uint4 qv = *reinterpret_cast<const uint4*>(q + off);
            if (r >= L) kv = qv = uint4{0u, 0u, 0u, 0u};
            *reinterpret_cast<uint4*>(&sK[r * XP + cv * VN]) = kv;
            *reinterpret_cast<uint4*>(&sQ[r * XP + cv * VN]) = qv;
        }
        if (tid < C) {
            const float bv = beta[((size_t)b * T + t0 + min(tid, L - 1)) * HV + h];
            sBeta[tid] = tid < L ? bv : 0.f;
        }
        for (int idx = tid; idx < C * AP; idx += 256) sT[idx] = 0.f;
    }
    __syncthreads();

    auto kval = [&](int r, int c) { return to_f32(sK[r * XP + c]); };
    auto qval = [&](int r, int c) { return to_f32(sQ[r * XP + c]); };
    auto gam = [&](int r, int c) { return sGam[r * GP + c]; };

    // ---- carry operands: decayed queries, decay-to-end keys (transposed), exp(gam_last) --
    for (int f = wave; f < NB * KC; f += 4) {
        const int rt = f / KC, p = f % KC;
        const int r = 16 * rt + li;
        half8 x;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int c = 32 * p + perm_slot(gq, jj);
            x[jj] = static_cast<_Float16>(qval(r, c) * __expf(gam(r, c)));
        }
        frags[(size_t)(R.off_qt + f) * 64 + lane] = x;
    }
    for (int f = wave; f < DKT * NQS; f += 4) {
        const int ct = f / NQS, qs = f % NQS;
        const int c = 16 * ct + li;
        const float gl = gam(C - 1, c);
        half8 x;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int r = 32 * qs + perm_slot(gq, jj);
            x[jj] = r < C ? static_cast<_Float16>(kval(r, c) * __expf(gl - gam(r, c)))
                          : static_cast<_Float16>(0.f);
        }
        frags[(size_t)(R.off_kb + f) * 64 + lane] = x;
    }
    if (tid < DK) egl_out[tid] = __expf(gam(C - 1, tid));

    // ---- gram A (-> LDS, fp32) and causal terms P (-> fragments), wave I = row block ----
    if (wave < NB) {
        const int I = wave;
        const int r = 16 * I + li;  // B-operand row (query/key side)
        f32x4 Pt[NB];
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            f32x4 accA = {0.f, 0.f, 0.f, 0.f};
            f32x4 accP = {0.f, 0.f, 0.f, 0.f};
            const int s = 16 * J + li;  // A-operand row (key side)
            if (J < I) {
                const int m = 16 * J + 15;
#pragma unroll
                for (int p = 0; p < KC; ++p) {
                    half8 a, bk, bq;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int c = 32 * p + 8 * gq + jj;
                        const float gm = gam(m, c);
                        a[jj] = static_cast<_Float16>(kval(s, c) * __expf(gm - gam(s, c)));
                        const float fr = __expf(gam(r, c) - gm);
                        bk[jj] = static_cast<_Float16>(kval(r, c) * fr);
                        bq[jj] = static_cast<_Float16>(qval(r, c) * fr);
                    }
                    accA = mfma_f16(a, bk, accA);
                    accP = mfma_f16(a, bq, accP);
                }
            } else if (J == I) {
                const int m = 16 * I + 7;
#pragma unroll
                for (int p = 0; p < KC; ++p) {
                    bf16x8 ah, al, kh_, kl, qh, ql;
#pragma unroll
                    for (int jj = 0; jj < 8; ++jj) {
                        const int c = 32 * p + 8 * gq + jj;
                        const float gm = gam(m, c);
                        __bf16 hi, lo;
                        split_bf16(kval(s, c) * __expf(gm - gam(s, c)), hi, lo);
                        ah[jj] = hi;
                        al[jj] = lo;
                        const float fr = __expf(gam(r, c) - gm);
                        split_bf16(kval(r, c) * fr, hi, lo);
                        kh_[jj] = hi;
                        kl[jj] = lo;
                        split_bf16(qval(r, c) * fr, hi, lo);
                        qh[jj] = hi;
                        ql[jj] = lo;
                    }
                    accA = mfma_bf16(ah, kh_, accA);
                    accA = mfma_bf16(al, kh_, accA);
                    accA = mfma_bf16(ah, kl, accA);
                    accP = mfma_bf16(ah, qh, accP);
                    accP = mfma_bf16(al, qh, accP);
                    accP = mfma_bf16(ah, ql, accP);
                }
            }
            // accumulator lane holds [s = 16J + 4gq + i][r = 16I + li]
            const float br = sBeta[r];
            f32x4 av, pv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int sl = 4 * gq + i;
                const bool lowA = J < I || (J == I && sl < li);
                const bool lowP = J < I || (J == I && sl <= li);
                av[i] = lowA ? accA[i] * br : 0.f;
                pv[i] = lowP ? accP[i] : 0.f;
            }
            if (J <= I) *reinterpret_cast<f32x4*>(&sA[r * AP + 16 * J + 4 * gq]) = av;
            Pt[J] = (J <= I) ? pv : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // P fragments for row block I: slot jj <- tile J = 2qs + jj/4, row i = jj % 4
        // (token steps qs <= I/2 only; the rest of the block row is zero)
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
            if (2 * qs > I) break;
            half8 x;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int J = 2 * qs + (jj >> 2);
                x[jj] = J < NB ? static_cast<_Float16>(Pt[J < NB ? J : 0][jj & 3])
                               : static_cast<_Float16>(0.f);
            }
            frags[(size_t)(R.off_p + ChunkRecord::tri_base(I) + qs) * 64 + lane] = x;
        }
    } else {
        // rows of A above the computed blocks are never read; nothing to do
    }
    __syncthreads();

    // ---- block forward substitution: Tinv = (I + A)^-1 ---------------------------------
    // diagonal 16x16 blocks: lane j of wave w inverts column j of block w
    if (wave < NB && lane < 16) {
        const int base = 16 * wave;
        const int j = lane;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == j) ? 1.f : 0.f;
#pragma unroll
            for (int kk = 0; kk < i; ++kk) s -= sA[(base + i) * AP + base + kk] * x[kk];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sT[(base + i) * AP + base + j] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks by distance d:  Tinv_IJ = -Tinv_II * sum_{M=J}^{I-1} A_IM Tinv_MJ
#pragma unroll
    for (int d = 1; d < NB; ++d) {
        const int ii = tid >> 4, jj = tid & 15;
        for (int I = d; I < NB; ++I) {
            const int J = I - d;
            float y = 0.f;
            for (int M = J; M < I; ++M)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    y += sA[(16 * I + ii) * AP + 16 * M + kk] * sT[(16 * M + kk) * AP + 16 * J + jj];
            sY[(I - d) * 256 + tid] = y;
        }
        __syncthreads();
        for (int I = d; I < NB; ++I) {
            const int J = I - d;
            float t = 0.f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
                t -= sT[(16 * I + ii) * AP + 16 * I + kk] * sY[(I - d) * 256 + kk * 16 + jj];
            sT[(16 * I + ii) * AP + 16 * J + jj] = t;
        }
        __syncthreads();
    }

    // ---- Tb = Tinv diag(beta) fragments ------------------------------------------------
    for (int f = wave; f < NB * NQS; f += 4) {
        const int rt = f / NQS, qs = f % NQS;
        if (2 * qs > rt) continue;
        const int r = 16 * rt + li;
        half8 x;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int s = 32 * qs + perm_slot(gq, jj);
            x[jj] = s < C ? static_cast<_Float16>(sT[r * AP + s] * sBeta[s])
                          : static_cast<_Float16>(0.f);
        }
        frags[(size_t)(R.off_tb + ChunkRecord::tri_base(rt) + qs) * 64 + lane] = x;
    }

    // ---- pseudo-keys: W^T = (exp(gam) * K)^T Tb^T on the matrix cores; store -W --------
    if (wave < KC) {
        const int p = wave;
        half8 ka[2][NQS];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
            const int c = 16 * (2 * p + h2) + li;
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int s = 32 * qs + 8 * gq + jj;
                    ka[h2][qs][jj] = s < C ? static_cast<_Float16>(kval(s, c) * __expf(gam(s, c)))
                                           : static_cast<_Float16>(0.f);
                }
            }
        }
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
            f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
            const int r = 16 * rt + li;
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
                if (2 * qs > rt) break;
                half8 bt;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int s = 32 * qs + 8 * gq + jj;
                    bt[jj] = s < C ? static_cast<_Float16>(sT[r * AP + s] * sBeta[s])
                                   : static_cast<_Float16>(0.f);
                }
                acc0 = mfma_f16(ka[0][qs], bt, acc0);
                acc1 = mfma_f16(ka[1][qs], bt, acc1);
            }
            half8 x;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj)
                x[jj] = static_cast<_Float16>(-((jj >> 2) ? acc1[jj & 3] : acc0[jj & 3]));
            frags[(size_t)(R.off_w + rt * KC + p) * 64 + lane] = x;
        }
    }
}

template <typename TIn, int DK, int C>
static hipError_t launch_prep_t(const LaunchArgs& a) {
    const int NC = (a.T + C - 1) / C;
    const long long nblk = (long long)a.B * a.HV * NC;
    hipLaunchKernelGGL((chunk_prep_kernel<TIn, DK, C>), dim3((unsigned)nblk), dim3(256), 0,
                       (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, a.g, a.beta,
                       (unsigned char*)a.workspace, a.T, a.HK, a.HV, NC);
    return hipGetLastError();
}

template <typename TIn>
static hipError_t dispatch_prep(const LaunchArgs& a) {
#define GDR_CASE(DK_, C_) \
    if (a.dk == DK_ && a.chunk == C_) return launch_prep_t<TIn, DK_, C_>(a);
    GDR_CASE(32, 16) GDR_CASE(32, 32) GDR_CASE(32, 64)
    GDR_CASE(64, 16) GDR_CASE(64, 32) GDR_CASE(64, 64)
    GDR_CASE(128, 16) GDR_CASE(128, 32) GDR_CASE(128, 64)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_prep(const LaunchArgs& a) {
    return a.qkv_f32 ? dispatch_prep<float>(a) : dispatch_prep<bf16_t>(a);
}

}  // namespace gdr

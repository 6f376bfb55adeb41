// Sequential half of the chunkwise WY/UT prefill: the inter-chunk state carry (gfx950).
//
// With the chunk operands prepared by chunk_prep (decayed queries Qt, pseudo-keys W,
// decay-to-end keys Kb, Tb = (I + A)^-1 diag(beta), causal terms P, exp(gam_last)), one
// chunk advances the state S (dk x dv) as
//   U    = Tb V - W S                  pseudo-values minus the state's prediction
//   O    = Qt S + P U                  outputs of the chunk's tokens
//   S'   = diag(exp(gam_last)) S + Kb^T U
// (ExecuTorch PR #21021 "Reorder channelwise gated delta rule chunked hot loops for
// autovectorization", second commit summary: WY pseudo-keys/values and inter-chunk state
// carry).  Columns of S evolve independently, so the value dimension is split across
// workgroups: one 64-lane wave owns NT 16-column tiles of one (batch, value head) and
// walks its chunks in order with the S tile resident in MFMA accumulators the whole time.
//
// Every product is a 16x16x32 fp16 MFMA with fp32 accumulation.  The accumulator tiles of
// S and U feed the B operand of the next product directly (the reduction slots follow
// perm_slot, which matches the rows an accumulator lane holds), so the carry needs no LDS
// and no cross-lane shuffles; the A operands arrive pre-permuted from the workspace.
//
// Launch: blocks = (B*HV) x (dv / (16*NT)), block index = colgroup * (B*HV) + head, so all
// column groups of a head share the same XCD (blocks are dealt round-robin to the 8 XCDs)
// and read the head's chunk operands from one L2.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {

template <typename TIn, int DK, int DV, int C, int NT>
__global__ __launch_bounds__(64) void chunk_carry_kernel(const TIn* __restrict__ v,
                                                         const float* h0, float* __restrict__ o,
                                                         float* ht,
                                                         const unsigned char* __restrict__ ws,
                                                         int B, int T, int HV, int NC) {
    constexpr int NB = C / 16;
    constexpr int NQS = (C + 31) / 32;
    constexpr int KC = DK / 32;
    constexpr int DKT = DK / 16;

    const ChunkRecord R = ChunkRecord::make(C, DK);
    const int NH = B * HV;
    const int blk = blockIdx.x;
    const int bh = blk % NH;
    const int cg = blk / NH;
    const int h = bh % HV;
    const int b = bh / HV;
    const int lane = threadIdx.x;
    const int li = lane & 15;
    const int gq = lane >> 4;

    int jcol[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) jcol[nt] = 16 * (cg * NT + nt) + li;

    // state tile in accumulator layout: S[ct][nt][i] = S[16ct + 4gq + i][jcol[nt]]
    f32x4 S[DKT][NT];
    const size_t sb = (size_t)bh * DK * DV;
#pragma unroll
    for (int ct = 0; ct < DKT; ++ct)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[ct][nt][i] = h0 ? h0[sb + (size_t)(16 * ct + 4 * gq + i) * DV + jcol[nt]] : 0.f;

    for (int n = 0; n < NC; ++n) {
        const unsigned char* rec = ws + (size_t)((size_t)bh * NC + n) * R.bytes;
        const half8* fr = reinterpret_cast<const half8*>(rec) + lane;
        const float* egl = reinterpret_cast<const float*>(rec + (size_t)R.nfrag * 1024);
        const int t0 = n * C;

        // B operands from the state accumulators
        half8 SB[KC][NT];
#pragma unroll
        for (int p = 0; p < KC; ++p)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj)
                    SB[p][nt][jj] = static_cast<_Float16>(S[2 * p + (jj >> 2)][nt][jj & 3]);

        // B operands from the chunk's values (rows past T are zero)
        half8 VB[NQS][NT];
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int r = 32 * qs + perm_slot(gq, jj);
                const int t = t0 + r;
                const bool live = r < C && t < T;
                const size_t vrow = (((size_t)b * T + (live ? t : 0)) * HV + h) * DV;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    VB[qs][nt][jj] = live ? static_cast<_Float16>(to_f32(v[vrow + jcol[nt]]))
                                          : static_cast<_Float16>(0.f);
            }

        // U = Tb V - W S
        f32x4 U[NB][NT];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) U[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
                if (2 * qs > rt) break;
                const half8 a = fr[(size_t)(R.off_tb + rt * NQS + qs) * 64];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) U[rt][nt] = mfma_f16(a, VB[qs][nt], U[rt][nt]);
            }
#pragma unroll
            for (int p = 0; p < KC; ++p) {
                const half8 a = fr[(size_t)(R.off_w + rt * KC + p) * 64];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) U[rt][nt] = mfma_f16(a, SB[p][nt], U[rt][nt]);
            }
        }

        // O = Qt S  (+ P U below)
        f32x4 O[NB][NT];
#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) O[rt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int p = 0; p < KC; ++p) {
                const half8 a = fr[(size_t)(R.off_qt + rt * KC + p) * 64];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) O[rt][nt] = mfma_f16(a, SB[p][nt], O[rt][nt]);
            }
        }

        // B operands from the U accumulators
        half8 UB[NQS][NT];
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int rt = 2 * qs + (jj >> 2);
                    UB[qs][nt][jj] = rt < NB ? static_cast<_Float16>(U[rt < NB ? rt : 0][nt][jj & 3])
                                             : static_cast<_Float16>(0.f);
                }

#pragma unroll
        for (int rt = 0; rt < NB; ++rt) {
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
                if (2 * qs > rt) break;
                const half8 a = fr[(size_t)(R.off_p + rt * NQS + qs) * 64];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) O[rt][nt] = mfma_f16(a, UB[qs][nt], O[rt][nt]);
            }
        }

        // S' = diag(exp(gam_last)) S + Kb^T U
#pragma unroll
        for (int ct = 0; ct < DKT; ++ct) {
            const f32x4 e = *reinterpret_cast<const f32x4*>(egl + 16 * ct + 4 * gq);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) S[ct][nt] *= e;
#pragma unroll
            for (int qs = 0; qs < NQS; ++qs) {
                const half8 a = fr[(size_t)(R.off_kb + ct * NQS + qs) * 64];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) S[ct][nt] = mfma_f16(a, UB[qs][nt], S[ct][nt]);
            }
        }

        // outputs: rows 16rt + 4gq + i of this chunk
#pragma unroll
        for (int rt = 0; rt < NB; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = t0 + 16 * rt + 4 * gq + i;
                if (t < T) {
                    const size_t orow = (((size_t)b * T + t) * HV + h) * DV;
#pragma unroll
                    for (int nt = 0; nt < NT; ++nt) o[orow + jcol[nt]] = O[rt][nt][i];
                }
            }
    }

    if (ht) {
#pragma unroll
        for (int ct = 0; ct < DKT; ++ct)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ht[sb + (size_t)(16 * ct + 4 * gq + i) * DV + jcol[nt]] = S[ct][nt][i];
    }
}

template <typename TIn, int DK, int DV, int C, int NT>
static hipError_t launch_carry_t(const LaunchArgs& a) {
    const int NC = (a.T + C - 1) / C;
    const long long nblk = (long long)a.B * a.HV * (DV / (16 * NT));
    hipLaunchKernelGGL((chunk_carry_kernel<TIn, DK, DV, C, NT>), dim3((unsigned)nblk), dim3(64), 0,
                       (hipStream_t)a.stream, (const TIn*)a.v, a.h0, a.o, a.ht,
                       (const unsigned char*)a.workspace, a.B, a.T, a.HV, NC);
    return hipGetLastError();
}

template <typename TIn, int DK, int DV>
static hipError_t dispatch_chunk(const LaunchArgs& a) {
    if (a.chunk == 16) return launch_carry_t<TIn, DK, DV, 16, 1>(a);
    if (a.chunk == 32) return launch_carry_t<TIn, DK, DV, 32, 1>(a);
    if (a.chunk == 64) return launch_carry_t<TIn, DK, DV, 64, 1>(a);
    return hipErrorInvalidValue;
}

template <typename TIn>
static hipError_t dispatch_carry(const LaunchArgs& a) {
#define GDR_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return dispatch_chunk<TIn, DK_, DV_>(a);
    GDR_CASE(32, 32) GDR_CASE(32, 64) GDR_CASE(32, 128)
    GDR_CASE(64, 32) GDR_CASE(64, 64) GDR_CASE(64, 128)
    GDR_CASE(128, 32) GDR_CASE(128, 64) GDR_CASE(128, 128)
#undef GDR_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_carry(const LaunchArgs& a) {
    return a.qkv_f32 ? dispatch_carry<float>(a) : dispatch_carry<bf16_t>(a);
}

}  // namespace gdr

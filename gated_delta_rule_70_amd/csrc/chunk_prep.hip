// Chunk-parallel half of the chunkwise WY/UT prefill (gfx950).
//
// ExecuTorch PR #21021 ("Reorder channelwise gated delta rule chunked hot loops for
// autovectorization", second commit summary) evaluates prefill chunk by chunk: per-channel
// log-decay prefixes, the beta-folded triangular transform, WY pseudo-keys and
// pseudo-values, causal query/key terms, then the inter-chunk state carry.  Everything
// except the carry depends on one chunk only, so this kernel runs it for all
// (batch, value head, chunk) triples in parallel -- persistent 512-thread workgroups, one
// item at a time each -- and hands the results to the sequential carry kernel as fp16 MFMA
// operand fragments.
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
// Decay factors.  Every factor is built from two per-element exponentials around the
// middle row m_I = 16I + 7 of the element's 16-row block I,
//   Z_rc = exp(gam_rc - gam_{m_I,c}),   Zi_rc = exp(gam_{m_I,c} - gam_rc),
// and per-(block, channel) constants, so no operand leaves its format's range:
//   blocks J < I (fp16):  exp(gam_r - gam_s) = [Z_r a_I] [Zi_s b_J] E_IJ, where
//       a_I = exp(gam_m - gam_{16I-1}), b_J = exp(gam_{16J+15} - gam_m),
//       E_IJ = exp(gam_{16I-1} - gam_{16J+15}); both bracketed factors are <= 1;
//   diagonal blocks (bf16 hi + lo split, three products, fp32 range, ~16 bits):
//       exp(gam_r - gam_s) = Z_r Zi_s;
//   Qt = q Z G_I, Kb = k Zi L_I, exp(gam) k = k Z G_I with G_I = exp(gam_m),
//       L_I = exp(gam_last - gam_m).
// Z and Zi stay finite while the decay over 8 consecutive tokens of a block is below ~88
// (mean g above about -11 per token), the range documented in gdr.h.
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
__global__ __launch_bounds__(512) void chunk_prep_kernel(const TIn* __restrict__ q,
                                                         const TIn* __restrict__ k,
                                                         const float* __restrict__ g,
                                                         const float* __restrict__ beta,
                                                         unsigned char* __restrict__ ws, int B,
                                                         int T, int HK, int HV, int NC) {
    constexpr int NTH = 512;
    constexpr int NB = C / 16;
    constexpr int NQS = (C + 31) / 32;
    constexpr int KC = DK / 32;
    constexpr int DKT = DK / 16;
    constexpr int ZP = DK + 4;        // padded fp32 row (Z, Zi)
    constexpr int VN = VecLoad<TIn>::N;
    constexpr int XP = DK + VN;       // padded input row (k)
    constexpr int AP = C + 4;         // padded fp32 row (A, Tinv)
    constexpr int NSEG = NTH / DK;    // scan segments per channel
    constexpr int RPS = C / NSEG;     // rows per segment
    constexpr int NOFF = NB * (NB - 1) / 2;
    static_assert(RPS >= 1 && C % NSEG == 0, "chunk too short for this key dim");
    constexpr ChunkRecord R = ChunkRecord::make(C, DK);

    // LDS.  Z/Zi are dead once the gram and the carry operands are formed; Tinv reuses them.
    constexpr int NZZ = (2 * C * ZP > C * AP) ? 2 * C * ZP : C * AP;
    __shared__ float sZZ[NZZ];
    __shared__ TIn sK[C * XP];
    __shared__ float sA[C * AP];
    __shared__ _Float16 sP[C * C];
    __shared__ float sRef[NB * 3 * DK];      // gam at rows 16I-1, 16I+7, 16I+15
    __shared__ float sCa[NB * DK], sCb[NB * DK], sCg[NB * DK], sCl[NB * DK];
    __shared__ float sCe[(NOFF > 0 ? NOFF : 1) * DK];
    __shared__ float sSeg[NSEG * DK];
    __shared__ float sBeta[C];
    __shared__ float sY[(NB > 1 ? NB - 1 : 1) * 256];
    float* sZ = sZZ;
    float* sZi = sZZ + C * ZP;
    float* sT = sZZ;  // Tinv reuses the Z/Zi area once the gram is done

    const int tid0 = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int sc = tid0 % DK;     // channel of this thread in the scan
    const int sseg = tid0 / DK;   // segment of this thread
    constexpr int VPR = DK / VN;                       // k vectors per row
    constexpr int KV = (C * VPR + NTH - 1) / NTH;      // k vectors per thread

    // Persistent workgroups: each walks (batch, head, chunk) items with a stride of the
    // grid and prefetches the next item's g, k and beta into registers while the current
    // item computes, so neither a workgroup launch nor the input latency sits between items.
    const int total = B * HV * NC;
    float gpre[RPS];
    uint4 kpre[KV];
    float bpre = 0.f;
    auto prefetch = [&](int it) {
        const int pn = it % NC, pbh = it / NC;
        const int ph = pbh % HV, pb = pbh / HV, pkh = ph / (HV / HK);
        const int pt0 = pn * C, pL = min(C, T - pt0);
#pragma unroll
        for (int m = 0; m < RPS; ++m) {  // unconditional loads from clamped rows, masked later
            const int r = sseg * RPS + m;
            gpre[m] = g[(((size_t)pb * T + pt0 + min(r, pL - 1)) * HV + ph) * DK + sc];
        }
        const size_t prow0 = (((size_t)pb * T + pt0) * HK + pkh) * DK;
#pragma unroll
        for (int i = 0; i < KV; ++i) {
            const int idx = tid0 + i * NTH;
            const int r = idx / VPR, cv = idx % VPR;
            if (idx < C * VPR)
                kpre[i] = *reinterpret_cast<const uint4*>(k + prow0 + min(r, pL - 1) * (size_t)HK * DK + cv * VN);
        }
        if (tid0 < C) bpre = beta[((size_t)pb * T + pt0 + min(tid0, pL - 1)) * HV + ph];
    };
    if (blockIdx.x < total) prefetch(blockIdx.x);

    for (int item = blockIdx.x; item < total; item += gridDim.x) {
    // Lane indices are laundered through an empty asm each iteration: otherwise the
    // compiler hoists every per-lane LDS address of the (fully unrolled) body out of the
    // loop and keeps them all live, which overflows the register file.
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;
    const int n = item % NC;
    const int bh = item / NC;
    const int h = bh % HV;
    const int b = bh / HV;
    const int kh = h / (HV / HK);
    const int t0 = n * C;
    const int L = min(C, T - t0);

    unsigned char* rec = ws + (size_t)((size_t)bh * NC + n) * R.bytes;
    half8* frags = reinterpret_cast<half8*>(rec);
    float* egl_out = reinterpret_cast<float*>(rec + (size_t)R.nfrag * 1024);
    const size_t qk_row0 = (((size_t)b * T + t0) * HK + kh) * DK;  // row r at qk_row0 + r*HK*DK
    const size_t qk_rstride = (size_t)HK * DK;

    // ---- 1. g -> per-channel inclusive prefix (two-level scan); k rows and beta -> LDS ----
    float gam_loc[RPS];
    {
        float acc = 0.f;
#pragma unroll
        for (int m = 0; m < RPS; ++m) {
            const int r = sseg * RPS + m;
            acc += r < L ? gpre[m] : 0.f;
            gam_loc[m] = acc;
        }
        sSeg[sseg * DK + sc] = acc;
#pragma unroll
        for (int i = 0; i < KV; ++i) {
            const int idx = tid + i * NTH;
            const int r = idx / VPR, cv = idx % VPR;
            if (idx < C * VPR) {
                const uint4 kv = r < L ? kpre[i] : uint4{0u, 0u, 0u, 0u};
                *reinterpret_cast<uint4*>(&sK[r * XP + cv * VN]) = kv;
            }
        }
        if (tid < C) sBeta[tid] = tid < L ? bpre : 0.f;
    }
    __syncthreads();
    {
        float off = 0.f;
        for (int s2 = 0; s2 < sseg; ++s2) off += sSeg[s2 * DK + sc];
#pragma unroll
        for (int m = 0; m < RPS; ++m) {
            const int r = sseg * RPS + m;
            const float gv = gam_loc[m] + off;
            gam_loc[m] = gv;
            const int I = r >> 4, rr = r & 15;
            if (rr == 7) sRef[(I * 3 + 1) * DK + sc] = gv;
            if (rr == 15) {
                sRef[(I * 3 + 2) * DK + sc] = gv;
                if (I + 1 < NB) sRef[((I + 1) * 3 + 0) * DK + sc] = gv;
            }
        }
        if (sseg == 0) sRef[0 * DK + sc] = 0.f;  // the row before the chunk: gam = 0
    }
    __syncthreads();
    // ---- 2. per-element factors Z, Zi and per-(block, channel) constants ----------------
    {
#pragma unroll
        for (int m = 0; m < RPS; ++m) {
            const int r = sseg * RPS + m;
            const int I = r >> 4;
            const float gm = sRef[(I * 3 + 1) * DK + sc];
            sZ[r * ZP + sc] = __expf(gam_loc[m] - gm);
            sZi[r * ZP + sc] = __expf(gm - gam_loc[m]);
        }
        const float gl = sRef[((NB - 1) * 3 + 2) * DK + sc];  // gam at the last row
        for (int I = sseg; I < NB; I += NSEG) {
            const float gp = sRef[(I * 3 + 0) * DK + sc];
            const float gm = sRef[(I * 3 + 1) * DK + sc];
            const float ge = sRef[(I * 3 + 2) * DK + sc];
            sCa[I * DK + sc] = __expf(gm - gp);
            sCb[I * DK + sc] = __expf(ge - gm);
            sCg[I * DK + sc] = __expf(gm);
            sCl[I * DK + sc] = __expf(gl - gm);
        }
        for (int pr = sseg; pr < NOFF; pr += NSEG) {
            int I = 1, base = 0;
            while (base + I <= pr) base += I++;
            const int J = pr - base;
            sCe[pr * DK + sc] = __expf(sRef[(I * 3 + 0) * DK + sc] - sRef[(J * 3 + 2) * DK + sc]);
        }
        if (sseg == 0) egl_out[sc] = __expf(gl);
    }
    __syncthreads();

    auto kval = [&](int r, int c) { return to_f32(sK[r * XP + c]); };
    auto qrow = [&](int r) { return q + qk_row0 + min(r, L - 1) * qk_rstride; };
    // 4 consecutive q values of row r from channel c0 (zero past the chunk end)
    auto q4 = [&](int r, int c0, float (&x)[4]) {
        const TIn* p = qrow(r) + c0;
        if constexpr (VN == 8) {
            const uint2 u = *reinterpret_cast<const uint2*>(p);
            x[0] = __uint_as_float(u.x << 16);
            x[1] = __uint_as_float(u.x & 0xFFFF0000u);
            x[2] = __uint_as_float(u.y << 16);
            x[3] = __uint_as_float(u.y & 0xFFFF0000u);
        } else {
            const float4 u = *reinterpret_cast<const float4*>(p);
            x[0] = u.x; x[1] = u.y; x[2] = u.z; x[3] = u.w;
        }
        if (r >= L) x[0] = x[1] = x[2] = x[3] = 0.f;
    };
    // 8 consecutive q values of row r from channel c0 (zero past the chunk end)
    auto q8 = [&](int r, int c0, float (&x)[8]) {
        const TIn* p = qrow(r) + c0;
        if constexpr (VN == 8) {
            const uint4 u = *reinterpret_cast<const uint4*>(p);
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[2 * j] = __uint_as_float(w4[j] << 16);
                x[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
            }
        } else {
            const float4 u0 = *reinterpret_cast<const float4*>(p);
            const float4 u1 = *reinterpret_cast<const float4*>(p + 4);
            x[0] = u0.x; x[1] = u0.y; x[2] = u0.z; x[3] = u0.w;
            x[4] = u1.x; x[5] = u1.y; x[6] = u1.z; x[7] = u1.w;
        }
        if (r >= L) {
#pragma unroll
            for (int j = 0; j < 8; ++j) x[j] = 0.f;
        }
    };

    // ---- 3. carry operands: Qt and Kb^T fragments; exp(gam) k fragments for W ------------
    static_assert((NB * KC) % (NTH / 64) == 0 || NB * KC < NTH / 64, "Qt fragments per wave");
    constexpr int QT_PER_WAVE = (NB * KC + NTH / 64 - 1) / (NTH / 64);
    float qx[QT_PER_WAVE][4], qy[QT_PER_WAVE][4];  // all q loads issued first
#pragma unroll
    for (int i = 0; i < QT_PER_WAVE; ++i) {
        const int f = wave + i * (NTH / 64);
        if (f < NB * KC) {
            const int rt = f / KC, p = f % KC;
            q4(16 * rt + li, 32 * p + 4 * gq, qx[i]);       // slots 0..3: channels 32p + 4gq + 0..3
            q4(16 * rt + li, 32 * p + 16 + 4 * gq, qy[i]);  // slots 4..7: channels 32p + 16 + 4gq + ..
        }
    }
#pragma unroll
    for (int i = 0; i < QT_PER_WAVE; ++i) {
        const int f = wave + i * (NTH / 64);
        if (f >= NB * KC) break;
        const int rt = f / KC, p = f % KC;
        const int r = 16 * rt + li;
        const float (&x)[4] = qx[i];
        const float (&y)[4] = qy[i];
        half8 o8;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int c = 32 * p + perm_slot(gq, jj);
            const float qv = jj < 4 ? x[jj] : y[jj - 4];
            o8[jj] = static_cast<_Float16>(qv * sZ[r * ZP + c] * sCg[rt * DK + c]);
        }
        frags[(size_t)(R.off_qt + f) * 64 + lane] = o8;
    }
    for (int f = wave; f < DKT * NQS; f += NTH / 64) {
        const int ct = f / NQS, qs = f % NQS;
        const int c = 16 * ct + li;
        half8 o8;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int r = 32 * qs + perm_slot(gq, jj);
            o8[jj] = r < C ? static_cast<_Float16>(kval(r, c) * sZi[r * ZP + c] * sCl[(r >> 4) * DK + c])
                           : static_cast<_Float16>(0.f);
        }
        frags[(size_t)(R.off_kb + f) * 64 + lane] = o8;
    }
    // W^T = (exp(gam) K)^T Tb^T is computed by wave w for key-channel step p = w % KC and
    // row tiles rt = w / KC, w / KC + 8 / KC, ...; its A operand (exp(gam) k, transposed)
    // is formed now, while Z is still live.
    constexpr int WW = (NTH / 64) / KC;  // waves per key-channel step (2, 4 or 8)
    const int wp = wave % KC;
    half8 ka[2][NQS];
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
        const int c = 16 * (2 * wp + h2) + li;
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int s = 32 * qs + 8 * gq + jj;
                ka[h2][qs][jj] = s < C ? static_cast<_Float16>(kval(s, c) * sZ[s * ZP + c] * sCg[(s >> 4) * DK + c])
                                       : static_cast<_Float16>(0.f);
            }
    }

    // ---- 4. gram A (-> sA, fp32, times beta_r) and causal terms P (-> sP, fp16) ---------
    // Work items: the NB diagonal block pairs first (three bf16 products per step), then the
    // NB(NB-1)/2 off-diagonal pairs (one fp16 product per step), dealt round-robin to waves.
    // The accumulator holds the transposed tile [s in block J][r in block I].
    for (int item = wave; item < NB + NOFF; item += NTH / 64) {
        int I, J, pr = -1;
        if (item < NB) {
            I = J = item;
        } else {
            pr = item - NB;
            I = 1;
            int base = 0;
            while (base + I <= pr) base += I++;
            J = pr - base;
        }
        const int s = 16 * J + li;  // A-operand row (key side)
        const int r = 16 * I + li;  // B-operand row (key / query side)
        f32x4 accA = {0.f, 0.f, 0.f, 0.f};
        f32x4 accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < KC; ++p) {
            const int c0 = 32 * p + 8 * gq;
            float qv[8];
            q8(r, c0, qv);
            if (I == J) {
                bf16x8 ah, al, kh_, kl, qh, ql;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int c = c0 + jj;
                    __bf16 hi, lo;
                    split_bf16(kval(s, c) * sZi[s * ZP + c], hi, lo);
                    ah[jj] = hi;
                    al[jj] = lo;
                    const float z = sZ[r * ZP + c];
                    split_bf16(kval(r, c) * z, hi, lo);
                    kh_[jj] = hi;
                    kl[jj] = lo;
                    split_bf16(qv[jj] * z, hi, lo);
                    qh[jj] = hi;
                    ql[jj] = lo;
                }
                accA = mfma_bf16(ah, kh_, accA);
                accA = mfma_bf16(al, kh_, accA);
                accA = mfma_bf16(ah, kl, accA);
                accP = mfma_bf16(ah, qh, accP);
                accP = mfma_bf16(al, qh, accP);
                accP = mfma_bf16(ah, ql, accP);
            } else {
                half8 a, bk, bq;
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int c = c0 + jj;
                    a[jj] = static_cast<_Float16>(kval(s, c) * sZi[s * ZP + c] * sCb[J * DK + c] * sCe[pr * DK + c]);
                    const float za = sZ[r * ZP + c] * sCa[I * DK + c];
                    bk[jj] = static_cast<_Float16>(kval(r, c) * za);
                    bq[jj] = static_cast<_Float16>(qv[jj] * za);
                }
                accA = mfma_f16(a, bk, accA);
                accP = mfma_f16(a, bq, accP);
            }
        }
        const float br = sBeta[r];
        f32x4 av;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int sl = 4 * gq + i;
            const bool lowA = J < I || sl < li;
            const bool lowP = J < I || sl <= li;
            av[i] = lowA ? accA[i] * br : 0.f;
            sP[r * C + 16 * J + sl] = static_cast<_Float16>(lowP ? accP[i] : 0.f);
        }
        *reinterpret_cast<f32x4*>(&sA[r * AP + 16 * J + 4 * gq]) = av;
    }
    __syncthreads();  // gram done; Z, Zi no longer needed

    // ---- 5. P fragments (block lower triangle) and Tinv := 0 ----------------------------
    for (int f = wave; f < R.ntri; f += NTH / 64) {
        int rt = 0;
        while (ChunkRecord::tri_base(rt + 1) <= f) ++rt;
        const int qs = f - ChunkRecord::tri_base(rt);
        const int r = 16 * rt + li;
        half8 x;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int sx = 32 * qs + perm_slot(gq, jj);
            x[jj] = (sx < C && sx <= r) ? sP[r * C + sx] : static_cast<_Float16>(0.f);
        }
        frags[(size_t)(R.off_p + f) * 64 + lane] = x;
    }
    for (int idx = tid; idx < C * AP; idx += NTH) sT[idx] = 0.f;
    __syncthreads();

    // ---- 6. block forward substitution: Tinv = (I + A)^-1 ------------------------------
    // diagonal 16x16 blocks, all at once: lane 16*blk + j of wave 0 solves column j of
    // block blk by substitution down its 16 rows.
    if (wave == 0 && (lane >> 4) < NB) {
        const int base = 16 * (lane >> 4);
        const int j = lane & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            asm volatile("" ::: "memory");  // load row i just before use (bounds register use)
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
        const int e = tid & 255, ii = e >> 4, jj = e & 15;
        for (int I = d + (tid >> 8); I < NB; I += NTH / 256) {
            const int J = I - d;
            float y = 0.f;
            for (int M = J; M < I; ++M)
#pragma unroll
                for (int kk = 0; kk < 16; ++kk)
                    y += sA[(16 * I + ii) * AP + 16 * M + kk] * sT[(16 * M + kk) * AP + 16 * J + jj];
            sY[(I - d) * 256 + e] = y;
        }
        __syncthreads();
        for (int I = d + (tid >> 8); I < NB; I += NTH / 256) {
            const int J = I - d;
            float t = 0.f;
#pragma unroll
            for (int kk = 0; kk < 16; ++kk)
                t -= sT[(16 * I + ii) * AP + 16 * I + kk] * sY[(I - d) * 256 + kk * 16 + jj];
            sT[(16 * I + ii) * AP + 16 * J + jj] = t;
        }
        __syncthreads();
    }

    // the next item's inputs: issued here (register pressure is low from now on) and
    // landing while this item finishes
    if (item + (int)gridDim.x < total) prefetch(item + gridDim.x);

    // ---- 7. Tb = Tinv diag(beta) fragments ----------------------------------------------
    for (int f = wave; f < R.ntri; f += NTH / 64) {
        int rt = 0;
        while (ChunkRecord::tri_base(rt + 1) <= f) ++rt;
        const int qs = f - ChunkRecord::tri_base(rt);
        const int r = 16 * rt + li;
        half8 x;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const int sx = 32 * qs + perm_slot(gq, jj);
            x[jj] = sx < C ? static_cast<_Float16>(sT[r * AP + sx] * sBeta[sx]) : static_cast<_Float16>(0.f);
        }
        frags[(size_t)(R.off_tb + f) * 64 + lane] = x;
    }

    // ---- 8. pseudo-keys: W^T = (exp(gam) K)^T Tb^T on the matrix cores; store -W --------
    for (int rt = wave / KC; rt < NB; rt += WW) {
        f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const int r = 16 * rt + li;
#pragma unroll
        for (int qs = 0; qs < NQS; ++qs) {
            if (2 * qs > rt) break;
            half8 bt;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int sx = 32 * qs + 8 * gq + jj;
                bt[jj] = sx < C ? static_cast<_Float16>(sT[r * AP + sx] * sBeta[sx]) : static_cast<_Float16>(0.f);
            }
            acc0 = mfma_f16(ka[0][qs], bt, acc0);
            acc1 = mfma_f16(ka[1][qs], bt, acc1);
        }
        half8 x;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            x[jj] = static_cast<_Float16>(-((jj >> 2) ? acc1[jj & 3] : acc0[jj & 3]));
        frags[(size_t)(R.off_w + rt * KC + wp) * 64 + lane] = x;
    }
    __syncthreads();  // the next item overwrites this item's LDS
    }
}

template <typename TIn, int DK, int C>
static hipError_t launch_prep_t(const LaunchArgs& a) {
    const int NC = (a.T + C - 1) / C;
    const long long items = (long long)a.B * a.HV * NC;
    // one persistent workgroup per resident slot (occupancy x CUs of the current device)
    static thread_local int cached_dev = -1, cached_slots = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
    if (dev != cached_dev) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return hipErrorInvalidDevice;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunk_prep_kernel<TIn, DK, C>, 512, 0) !=
            hipSuccess)
            return hipErrorInvalidDevice;
        cached_slots = cus * (per_cu > 0 ? per_cu : 1);
        cached_dev = dev;
    }
    const long long nblk = items < cached_slots ? items : cached_slots;
    hipLaunchKernelGGL((chunk_prep_kernel<TIn, DK, C>), dim3((unsigned)nblk), dim3(512), 0,
                       (hipStream_t)a.stream, (const TIn*)a.q, (const TIn*)a.k, a.g, a.beta,
                       (unsigned char*)a.workspace, a.B, a.T, a.HK, a.HV, NC);
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

// Tree-verify solve of the channelwise gated delta rule, gfx950.
//
// uzu PR #576 ("Support TreeUpdateSolve kernel") verifies a speculative token tree with a
// gram over the tree's tokens, a kh0 term (keys times the initial state) and an exact
// block triangular solve.  Here every node of a tree of T <= 64 tokens continues the
// recurrence from its parent's state (the parent of node t is parent[t] < t, -1 for the
// initial state h0) and its output is that of the plain recurrence along its root path.
// Unrolled along a path, that is the chunk algebra of one chunk with the causal order
// replaced by ancestry:
//   gam_t  = g_t + gam_parent(t)                   (decay prefix along the root path)
//   A_rs   = beta_r sum_c k_rc k_sc exp(gam_rc - gam_sc)   for s a strict ancestor of r
//   P_rs   =        sum_c q_rc k_sc exp(gam_rc - gam_sc)   for s = r or an ancestor of r
//   U      = (I + A)^-1 diag(beta) (V - (exp(gam) k) h0)  (forward substitution)
//   O      = (exp(gam) q) h0 + P U
// A and P are dot products of Kt = exp(gam) k (or Qt = exp(gam) q) with
// Kh = exp(-gam) k; every term that survives the ancestry mask is bounded by 1, the
// masked ones are finite while the path decay stays above -80 in every channel.
//
// One 256-thread workgroup per (batch, value head, 32-column block of v): the node-level
// terms live in LDS; the products run on the fp32 matrix cores (16x16x4); the forward
// substitution runs in one wave, its lanes split over columns and ancestor parity.
#include "gdr_device.h"
#include "gdr_launch.h"

namespace gdr {
namespace {

constexpr int TM = 64;  // most nodes per tree
constexpr int CB = 32;  // v columns per workgroup

// D(16x16) += A(16x4) B(4x16) in fp32.  Lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; D rows 4g .. 4g+3 of column l % 16 (g = l / 16).
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename TIn, int DK>
__global__ __launch_bounds__(256) void tree_verify_kernel(
    const int32_t* __restrict__ parent, const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ g, const float* __restrict__ beta,
    const float* __restrict__ h0, float* __restrict__ o, int T, int HK, int HV, int DV) {
    constexpr int KP = DK + 4;   // row pitch: lanes reading 16 rows at one column hit 16 banks
    constexpr int AP = TM + 4;
    constexpr int UP = CB + 4;
    __shared__ float sKt[TM * KP];  // gam, then exp(gam) k
    __shared__ float sKh[TM * KP];  // k, then exp(-gam) k
    __shared__ float sQt[TM * KP];  // q, then exp(gam) q
    __shared__ float sA[TM * AP];
    __shared__ float sP[TM * AP];
    __shared__ float sU[TM * UP];   // right-hand side, then U
    __shared__ int sPar[TM];
    __shared__ unsigned long long sAnc[TM];
    __shared__ float sBeta[TM];

    const int ncb = DV / CB;
    const int cb = blockIdx.x % ncb;
    const int bh = blockIdx.x / ncb;
    const int h = bh % HV;
    const int b = bh / HV;
    const int kh = h / (HV / HK);
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int li = lane & 15;
    const int gq = lane >> 4;
    const int T16 = (T + 15) & ~15;
    const int NB = T16 / 16;
    const int col0 = cb * CB;

    // ---- 0. parents (out-of-range entries read as -1), beta, raw g/k/q rows --------------
    for (int t = tid; t < TM; t += 256) {
        int p = -1;
        float bt = 0.f;
        if (t < T) {
            p = parent[(size_t)b * T + t];
            if (p < -1 || p >= t) p = -1;
            bt = beta[((size_t)b * T + t) * HV + h];
        }
        sPar[t] = p;
        sBeta[t] = bt;
    }
    for (int e = tid; e < T16 * DK; e += 256) {
        const int t = e / DK, c = e % DK;
        float gv = 0.f, kv = 0.f, qv = 0.f;
        if (t < T) {
            gv = g[(((size_t)b * T + t) * HV + h) * DK + c];
            kv = to_f32(k[(((size_t)b * T + t) * HK + kh) * DK + c]);
            qv = to_f32(q[(((size_t)b * T + t) * HK + kh) * DK + c]);
        }
        sKt[t * KP + c] = gv;
        sKh[t * KP + c] = kv;
        sQt[t * KP + c] = qv;
    }
    __syncthreads();

    // ---- 1. ancestor masks (walk up: parents are strictly smaller, so every walk ends) and
    //         decay prefixes along the root path (parents come first in each channel) ------
    if (tid < T) {
        unsigned long long m = 0;
        for (int r = sPar[tid]; r >= 0; r = sPar[r]) m |= 1ull << r;
        sAnc[tid] = m;
    }
    if (tid < DK) {
        for (int t = 1; t < T; ++t) {
            const int p = sPar[t];
            if (p >= 0) sKt[t * KP + tid] += sKt[p * KP + tid];
        }
    }
    __syncthreads();

    // ---- 2. decayed rows ---------------------------------------------------------------
    for (int e = tid; e < T16 * DK; e += 256) {
        const int i = (e / DK) * KP + e % DK;
        const float gm = sKt[i];
        const float kv = sKh[i];
        sKt[i] = __expf(gm) * kv;
        sKh[i] = __expf(-gm) * kv;
        sQt[i] *= __expf(gm);
    }
    __syncthreads();

    // ---- 3. A and P tiles on the matrix cores, masked by ancestry ------------------------
    // products: tile (I, J), J <= I, of A (x = 0) and P (x = 1); upper tiles are zero
    const int ntile = NB * NB;
    for (int job = wave; job < 2 * ntile; job += 4) {
        const int x = job / ntile;
        const int I = (job % ntile) / NB, J = (job % ntile) % NB;
        float* dst = x == 0 ? sA : sP;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (J <= I) {
            const float* ra = (x == 0 ? sKt : sQt) + (16 * I + li) * KP + gq;
            const float* rb = sKh + (16 * J + li) * KP + gq;
#pragma unroll 8
            for (int c = 0; c < DK; c += 4) acc = mfma4(ra[c], rb[c], acc);
        }
        const int s = 16 * J + li;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 16 * I + 4 * gq + i;
            float val = 0.f;
            if (J <= I && r < T && s < T) {
                const bool anc = (sAnc[r] >> s) & 1ull;
                if (x == 0) val = anc ? sBeta[r] * acc[i] : 0.f;
                else val = (anc || s == r) ? acc[i] : 0.f;
            }
            dst[r * AP + s] = val;
        }
    }

    // ---- 4. Kt h0 and Qt h0 for this column block; right-hand side beta (v - Kt h0) -------
    // tile (I, N): rows 16I.., columns col0 + 16N..; wave w owns tiles w, w+4, ... and keeps
    // its Qt h0 tiles for the output
    f32x4 qh[2];  // NB * 2 <= 8 tiles, at most 2 per wave
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = wave + 4 * u;
        f32x4 kacc = {0.f, 0.f, 0.f, 0.f}, qacc = {0.f, 0.f, 0.f, 0.f};
        if (tile < 2 * NB) {
            const int I = tile >> 1, N = tile & 1;
            if (h0 != nullptr) {
                const float* hb = h0 + ((size_t)bh * DK + gq) * DV + col0 + 16 * N + li;
                const float* ra = sKt + (16 * I + li) * KP + gq;
                const float* rq = sQt + (16 * I + li) * KP + gq;
#pragma unroll 8
                for (int c = 0; c < DK; c += 4) {
                    const float hv = hb[(size_t)c * DV];
                    kacc = mfma4(ra[c], hv, kacc);
                    qacc = mfma4(rq[c], hv, qacc);
                }
            }
            const int j = 16 * N + li;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * I + 4 * gq + i;
                float rhs = 0.f;
                if (r < T) {
                    const float vv = to_f32(v[(((size_t)b * T + r) * HV + h) * DV + col0 + j]);
                    rhs = sBeta[r] * (vv - kacc[i]);
                }
                sU[r * UP + j] = rhs;
            }
        }
        qh[u] = qacc;
    }
    __syncthreads();

    // ---- 5. forward substitution: U_r = rhs_r - sum_{s ancestor of r} A_rs U_s ------------
    // one wave: lane (j, half) sums the ancestors of parity `half` for column j
    if (wave == 0) {
        const int j = lane & (CB - 1);
        const int half = lane >> 5;
        for (int r = 1; r < T; ++r) {
            unsigned long long m = sAnc[r] & (half ? 0xAAAAAAAAAAAAAAAAull : 0x5555555555555555ull);
            float acc = 0.f;
            while (m) {
                const int s = __builtin_ctzll(m);
                m &= m - 1;
                acc += sA[r * AP + s] * sU[s * UP + j];
            }
            acc += __shfl_xor(acc, 32);
            if (half == 0) sU[r * UP + j] -= acc;
            // the next row reads this one: same wave, LDS accesses complete in order
        }
    }
    __syncthreads();

    // ---- 6. O = Qt h0 + P U ------------------------------------------------------------
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int tile = wave + 4 * u;
        if (tile < 2 * NB) {
            const int I = tile >> 1, N = tile & 1;
            f32x4 acc = qh[u];
            const float* rp = sP + (16 * I + li) * AP + gq;
            const float* ub = sU + gq * UP + 16 * N + li;
            for (int s = 0; s < T16; s += 4) acc = mfma4(rp[s], ub[s * UP], acc);
            const int col = col0 + 16 * N + li;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * I + 4 * gq + i;
                if (r < T) o[(((size_t)b * T + r) * HV + h) * DV + col] = acc[i];
            }
        }
    }
}

template <typename TIn, int DK>
hipError_t launch_tree_t(const LaunchArgs& a, const int32_t* parent) {
    const long long nblk = (long long)a.B * a.HV * (a.dv / CB);
    hipLaunchKernelGGL((tree_verify_kernel<TIn, DK>), dim3((unsigned)nblk), dim3(256), 0,
                       (hipStream_t)a.stream, parent, (const TIn*)a.q, (const TIn*)a.k,
                       (const TIn*)a.v, a.g, a.beta, a.h0, a.o, a.T, a.HK, a.HV, a.dv);
    return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch_tree(const LaunchArgs& a, const int32_t* parent) {
    if (a.dk == 32) return launch_tree_t<TIn, 32>(a, parent);
    if (a.dk == 64) return launch_tree_t<TIn, 64>(a, parent);
    if (a.dk == 128) return launch_tree_t<TIn, 128>(a, parent);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_tree_verify(const LaunchArgs& a, const int32_t* parent) {
    if (a.T < 1 || a.T > TM || a.dv % CB != 0) return hipErrorInvalidValue;
    return a.qkv_f32 ? dispatch_tree<float>(a, parent) : dispatch_tree<bf16_t>(a, parent);
}

}  // namespace gdr

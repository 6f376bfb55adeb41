// Internal interface between the host entry points (gdr_api.cpp) and the kernel launchers
// (one .hip file per kernel family).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdr {

// Largest group G = HV / HK the split prep form serves (its beta staging holds G rows).
constexpr int kSplitMaxGroup = 8;

struct LaunchArgs {
    int B, T, HK, HV, dk, dv, chunk;
    int HG;           // gate heads of g: HV (per value head) or HK (shared per key head)
    bool prep_split;  // prefill prep in split form (gate per key head, one workgroup per key head)
    bool qkv_f32;
    bool g_bf16;      // g stored as bf16 (only with bf16 q/k/v)
    bool k_l2norm;    // keys given raw: every kernel uses k / |k|_2 (fused prologue)
    bool g_softplus;  // g given as gate logits a: every kernel uses -softplus(a)
    bool o_bf16;      // o stored as bf16 (each fp32 output rounded to nearest even)
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const float* beta;
    const float* h0;
    void* o;          // fp32, or bf16 with o_bf16
    float* ht;
    void* workspace;
    void* stream;
    // Packed variable-length batch (nullptr / 0 for a dense [B][T] batch): B sequences laid
    // end to end in T rows, sequence b on rows [cu_seqlens[b], cu_seqlens[b + 1]).
    const int32_t* cu_seqlens;  // [B + 1], on the device
    int32_t* plan;              // prefill: the sequence plan in the workspace (VarlenPlan)
    int nct;                    // prefill: chunk slots, an upper bound on the sum of the
                                // sequences' chunk counts (varlen_chunk_slots)
};

// Largest number of sequences in one packed variable-length call (the plan kernel holds
// two entries per sequence in LDS).
constexpr int kVarlenMaxSeqs = 4096;

// Upper bound on sum_b ceil(len_b / C) over B sequences of T rows in all:
// ceil(len / C) <= (len + C - 1) / C, summed.
inline long long varlen_chunk_slots(long long B, long long T, int chunk) {
    return (T + B * (chunk - 1)) / chunk;
}

// The plan of a packed variable-length prefill, int32 in the workspace after the records:
//   [0, B]              sequence starts, sanitised: clamped to [0, T] and made
//                       non-decreasing (running maximum), so sequences never overlap
//   [B + 1, 2B + 1]     first chunk slot of each sequence (exclusive prefix of
//                       ceil(len / C)); entry 2B + 1 is the number of chunks in all
//   [2B + 2, 2B + 2 + nct)  the sequence of each chunk slot
// Chunk records are stored per sequence, then head, then chunk: sequence b's record of head
// h and chunk n sits at slot (first_b * HV + h * nchunks_b + n), which for a dense batch
// (first_b = b * NC, nchunks_b = NC) is the dense layout ((b * HV + h) * NC + n).
struct VarlenPlan {
    __host__ __device__ static constexpr long long ints(long long B, long long nct) { return 2 * (B + 1) + nct; }
    __host__ __device__ static constexpr int starts(int) { return 0; }
    __host__ __device__ static constexpr int first(int B) { return B + 1; }
    __host__ __device__ static constexpr int chunk_seq(int B) { return 2 * B + 2; }
};

// Rows and chunk records of batch element (dense) or sequence (packed) b: first row, rows,
// chunks, first chunk slot.
struct SeqSpan {
    long long row0;
    int T, nc, c0;
};
__device__ __forceinline__ SeqSpan seq_span(const int32_t* plan, int b, int B, int T, int NC) {
    if (plan == nullptr) return SeqSpan{(long long)b * T, T, NC, b * NC};
    const int r0 = plan[b], r1 = plan[b + 1];
    const int k0 = plan[VarlenPlan::first(B) + b], k1 = plan[VarlenPlan::first(B) + b + 1];
    return SeqSpan{r0, r1 - r0, k1 - k0, k0};
}

// Per-(batch, head, chunk) record that the chunk-parallel kernel writes and the
// sequential carry kernel reads: fp16 MFMA operand fragments (1 KiB each: 64 lanes x 8
// halves, lane-major) followed by one 1 KiB block of fp32 values: the chunk's total decay
// exp(gam_last) [dk], then the row multipliers [C] of Qt and [C] of P (the query rows are
// stored scaled by exact powers of two that keep them inside fp16's range; row r of the
// true Qt is the stored row times its multiplier, likewise for P).  Records are a whole
// number of KiB so the carry kernel can stream one into LDS with 1 KiB wave-wide copies.
//   Qt  [nb][kc]    decayed queries exp(gam) * q           (rows r, reduction over dk)
//   -W  [nb][kc]    negated WY pseudo-keys                  (rows r, reduction over dk)
//   Kb  [dkt][nqs]  decay-to-end keys, transposed           (rows c, reduction over tokens)
//   Tb  [nb][nqs]   Tinv diag(beta)                         (rows r, reduction over tokens)
//   P   [nb][nqs]   causal q.k terms                        (rows r, reduction over tokens)
// Tb and P are lower triangular: the slots of their all-zero fragments (token steps above
// a row tile's diagonal) are left unwritten, and the carry reads them as zeros from
// beyond the buffer range, so every row tile issues the same operand loads.
struct ChunkRecord {
    int nb;        // 16-row blocks per chunk (C / 16)
    int nqs;       // 32-wide token reduction steps (ceil(C / 32))
    int kc;        // 32-wide key-channel reduction steps (dk / 32)
    int dkt;       // 16-row key-channel tiles (dk / 16)
    int off_qt;    // fragment offsets (in fragments) of each operand
    int off_w;
    int off_kb;
    int off_tb;
    int off_p;
    int nfrag;     // operand fragments; the decay block follows them
    int bytes;     // record stride: (nfrag + 1) KiB
    int qsc;       // float offsets inside the decay block: Qt row multipliers [C]
    int psc;       //                                       P row multipliers [C]

    __host__ __device__ static constexpr ChunkRecord make(int C, int dk) {
        ChunkRecord r{};
        r.nb = C / 16;
        r.nqs = (C + 31) / 32;
        r.kc = dk / 32;
        r.dkt = dk / 16;
        r.off_qt = 0;
        r.off_w = r.off_qt + r.nb * r.kc;
        r.off_kb = r.off_w + r.nb * r.kc;
        r.off_tb = r.off_kb + r.dkt * r.nqs;
        r.off_p = r.off_tb + r.nb * r.nqs;
        r.nfrag = r.off_p + r.nb * r.nqs;
        r.bytes = (r.nfrag + 1) * 1024;
        r.qsc = dk;
        r.psc = dk + C;  // dk + 2C <= 256 floats for dk <= 128, C <= 64
        return r;
    }
};

// Workspace layout of the chunked prefill and the carry's plan.  The chunk records come
// first.  The whole-head carry (dk == dv in {64, 128}) is used where it beats the
// column-split one on an MI355X (256 compute units):
//   * more than 128 heads: one segment, one workgroup per head;
//   * heads whose 16-column tiles fit one round of 256 workgroups (heads * dv / 16 <= 256),
//     with enough chunks that the sequence can be cut into 256 / heads segments of at least
//     16 chunks each: that many segments, so ~256 workgroups carry at once.
// Between the two, the column split takes 2 or 4 tiles per workgroup and so still runs in
// one round.  (Carry right after the prep kernel at HV = 32, 128 x 128, chunk 64, whole
// head / column split: B = 8 T = 512 57 / 64 us; B = 1 T = 8192 215 / 221 us, T = 16384
// 371 / 408 us, T = 32768 704 / 779 us; B = 1 T = 4097, 8 segments of 8 chunks, 127 / 88 us;
// B = 2 T = 4097 (4 segments) 209 / 147 us, B = 4 T = 4097 (2 segments) 365 / 217 us,
// B = 3 T = 3000 263 / 143 us, B = 2 T = 8192 360 / 264 us.)  With more than one segment the
// workspace also holds each segment's summary [S_loc | M] (fp32, [heads][nseg - 1][2][dk]
// [dk]) and start state (fp32, [heads][nseg][dk][dv]).  A pure function of the dims, so
// the size query and the launch agree.
// A packed variable-length batch (varlen) never takes the time segments: its records are
// cnt slots per head (varlen_chunk_slots), followed by the plan (VarlenPlan).
struct CarryLayout {
    bool wide;
    int nseg;
    size_t rec_bytes, xsum_off, sstart_off, plan_off, total;
};

inline CarryLayout carry_layout(int B, int HV, int T, int dk, int dv, int chunk, bool varlen = false) {
    CarryLayout L{};
    const ChunkRecord R = ChunkRecord::make(chunk, dk);
    const long long NC = (T + (long long)chunk - 1) / chunk;
    const long long NH = (long long)B * HV;
    const long long slots = varlen ? varlen_chunk_slots(B, T, chunk) * HV : NH * NC;
    L.rec_bytes = (size_t)slots * (size_t)R.bytes;
    const bool dims_ok = dk == dv && (dk == 64 || dk == 128);
    L.nseg = 1;
    L.wide = false;
    if (dims_ok) {
        if (NH > 128) {
            L.wide = true;
        } else if (!varlen && NH * (dv / 16) <= 256) {
            const long long want = 256 / NH;  // >= 2
            if (NC >= 16 * want) {
                L.wide = true;
                L.nseg = (int)want;
            }
        }
    }
    const size_t mat = (size_t)dk * dk * 4;
    L.xsum_off = L.rec_bytes;
    L.sstart_off = L.xsum_off + (L.nseg > 1 ? (size_t)NH * (L.nseg - 1) * 2 * mat : 0);
    L.plan_off = L.sstart_off + (L.nseg > 1 ? (size_t)NH * L.nseg * mat : 0);
    L.total = L.plan_off +
              (varlen ? (size_t)VarlenPlan::ints(B, varlen_chunk_slots(B, T, chunk)) * 4 : 0);
    return L;
}

// Prep form for a gate shared per key head when the caller does not force one: the split
// form (a workgroup per key head and chunk, the gram computed once per group) once there
// are enough (batch element or sequence, key head, chunk) triples to fill the chip with it.  Measured on an
// MI355X at HK = 16, HV = 32, 128 x 128, chunk 64 (prep alone, fused / split): T = 512
// 15.6 / 18.0 us, T = 1024 21.9 / 19.1 us, T = 4097 62.2 / 57.8 us, T = 16384 249 / 202 us,
// B = 8 T = 512 58.2 / 49.9 us -- the split form wins from 256 triples.
inline bool split_prep_preferred(long long triples) { return triples >= 256; }

// packed variable-length prefill: sanitised starts and chunk plan into a.plan
hipError_t launch_varlen_plan(const LaunchArgs& a);
// token recurrence over a.T tokens in one launch (the decode step is a.T == 1; with
// a.cu_seqlens, over each packed sequence)
hipError_t launch_tokens(const LaunchArgs& a);
// The prep kernel in fused form (one workgroup per value head and chunk) or in split
// form (one per key head and chunk, solving per value head; needs HG == HK and
// HV / HK <= 8).
hipError_t launch_prep_fused(const LaunchArgs& a);
hipError_t launch_prep_split(const LaunchArgs& a);
inline hipError_t launch_chunk_prep(const LaunchArgs& a) {
    return a.prep_split ? launch_prep_split(a) : launch_prep_fused(a);
}
// the carry: whole-head segmented kernels where carry_layout says so, else the
// column-split kernel (launch_carry_split)
hipError_t launch_chunk_carry(const LaunchArgs& a);
hipError_t launch_carry_split(const LaunchArgs& a);
// tree-verify solve over trees of a.T <= 64 nodes; parent [B][T] int32 on the device
hipError_t launch_tree_verify(const LaunchArgs& a, const int32_t* parent);

}  // namespace gdr

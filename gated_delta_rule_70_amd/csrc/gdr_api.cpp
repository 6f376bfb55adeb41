// Host entry points of libgdr.so: argument validation, workspace sizing and kernel
// launches on the caller's stream.  Every check runs before the first HIP call, so a call
// that fails validation enqueues nothing and writes nothing.
#include "gdr.h"

#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "gdr_launch.h"

static_assert(gdr::kSplitMaxGroup == GDR_PREP_SPLIT_MAX_GROUP, "split prep group limit");
static_assert(gdr::kVarlenMaxSeqs == GDR_VARLEN_MAX_SEQS, "packed batch sequence limit");

// Workspace of the allocation-free prefill entry point (see gdr.h).  In host code `scratch`
// is only a handle to the device array; its address on a device comes from
// hipGetSymbolAddress, looked up once per device and cached.
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on a HIP error).
void* scratch_on_current_device() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool empty() const { return hi <= lo; }
};

Range range_of(const void* p, size_t bytes) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, p ? lo + bytes : lo};
}

bool overlap(Range a, Range b) { return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_head_dim(int d) { return d == 32 || d == 64 || d == 128; }

// Sizes in bytes of every tensor, computed in 64-bit with overflow checks.
struct Sizes {
    size_t q, v, g, beta, state, o;
};

// Multiply non-negative factors, failing on overflow past 2^62.
bool mul_ok(size_t a, size_t b, size_t* out) {
    if (a != 0 && b > (size_t(1) << 62) / a) return false;
    *out = a * b;
    return true;
}

// A packed variable-length batch (varlen) has its d.B sequences laid end to end in d.T token
// rows; the states are still one per sequence.
bool tensor_sizes(const gdr_dims& d, size_t elt, Sizes* s, bool varlen) {
    const size_t gelt = (d.flags & GDR_G_BF16) ? 2 : 4;
    size_t bt, bth, btv, x;
    if (!mul_ok(varlen ? 1 : (size_t)d.B, (size_t)d.T, &bt)) return false;
    if (!mul_ok(bt, (size_t)d.HK, &bth) || !mul_ok(bt, (size_t)d.HV, &btv)) return false;
    if (!mul_ok(bth, (size_t)d.dk, &x) || !mul_ok(x, elt, &s->q)) return false;
    if (!mul_ok(btv, (size_t)d.dv, &x) || !mul_ok(x, elt, &s->v)) return false;
    const size_t btg = (d.flags & GDR_G_PER_KEY_HEAD) ? bth : btv;  // g rows: key or value heads
    if (!mul_ok(btg, (size_t)d.dk, &x) || !mul_ok(x, gelt, &s->g)) return false;
    if (!mul_ok(btv, 4, &s->beta)) return false;
    const size_t oelt = (d.flags & GDR_O_BF16) ? 2 : 4;
    if (!mul_ok(btv, (size_t)d.dv, &x) || !mul_ok(x, oelt, &s->o)) return false;
    size_t bh;
    if (!mul_ok((size_t)d.B, (size_t)d.HV, &bh) || !mul_ok(bh, (size_t)d.dk, &x) ||
        !mul_ok(x, (size_t)d.dv, &x) || !mul_ok(x, 4, &s->state))
        return false;
    return true;
}

// Which entry point is validating: the decode step (T == 1), the fused token recurrence
// (any T, chunk ignored) or the chunked prefill (chunk checked).
enum class Path { decode, tokens, chunked };

// Shared validation of dims, pointers, alignment and aliasing.  `cu` is the sequence
// boundary array of a packed variable-length call (nullptr otherwise).
int validate(const gdr_dims* d, Path path, const void* q, const void* k, const void* v,
             const void* g, const float* beta, const float* h0, const void* o,
             const float* ht, Sizes* sizes, const int32_t* cu = nullptr, bool varlen = false) {
    if (!d || !q || !k || !v || !g || !beta || !o || (varlen && !cu)) return GDR_ERR_NULL;
    if (d->B < 1 || d->T < 1 || d->HK < 1 || d->HV < 1 || d->HV % d->HK != 0) return GDR_ERR_SHAPE;
    if (varlen && d->B > GDR_VARLEN_MAX_SEQS) return GDR_ERR_SHAPE;
    if (path == Path::decode && d->T != 1) return GDR_ERR_SHAPE;
    if (!supported_head_dim(d->dk) || !supported_head_dim(d->dv)) return GDR_ERR_UNSUPPORTED;
    if (d->qkv_dtype != GDR_BF16 && d->qkv_dtype != GDR_F32) return GDR_ERR_UNSUPPORTED;
    constexpr int32_t known = GDR_G_BF16 | GDR_K_L2NORM | GDR_G_SOFTPLUS | GDR_G_PER_KEY_HEAD |
                              GDR_PREP_SPLIT | GDR_PREP_FUSED | GDR_O_BF16;
    if ((d->flags & ~known) != 0) return GDR_ERR_UNSUPPORTED;
    if ((d->flags & GDR_G_BF16) && d->qkv_dtype != GDR_BF16) return GDR_ERR_UNSUPPORTED;
    if ((d->flags & GDR_PREP_SPLIT) &&
        ((d->flags & GDR_PREP_FUSED) || !(d->flags & GDR_G_PER_KEY_HEAD) ||
         d->HV / d->HK > GDR_PREP_SPLIT_MAX_GROUP))
        return GDR_ERR_UNSUPPORTED;
    if (path == Path::chunked && d->chunk != 16 && d->chunk != 32 && d->chunk != 64)
        return GDR_ERR_UNSUPPORTED;
    const size_t elt = d->qkv_dtype == GDR_F32 ? 4 : 2;
    if (!tensor_sizes(*d, elt, sizes, varlen)) return GDR_ERR_SHAPE;
    // Grid sizes must fit the launch limits: (B*HV) heads times chunks or column tiles; a
    // packed batch's prep covers its chunk slots per value head (plus a partial run of 8).
    const long long heads = (long long)d->B * d->HV;
    long long grid = heads * (path == Path::chunked && !varlen ? ((long long)d->T + d->chunk - 1) / d->chunk : 1);
    if (path == Path::chunked && varlen) grid = (gdr::varlen_chunk_slots(d->B, d->T, d->chunk) + 8) * d->HV;
    if (grid >= (1LL << 31) || heads * (d->dv / 16) >= (1LL << 31)) return GDR_ERR_SHAPE;

    const void* ptrs[] = {q, k, v, g, beta, h0, o, ht};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDR_ERR_ALIGN;
    if (cu && (reinterpret_cast<uintptr_t>(cu) & 3u) != 0) return GDR_ERR_ALIGN;

    const Range rq = range_of(q, sizes->q), rk = range_of(k, sizes->q), rv = range_of(v, sizes->v),
                rg = range_of(g, sizes->g), rb = range_of(beta, sizes->beta),
                rh0 = range_of(h0, sizes->state), ro = range_of(o, sizes->o),
                rht = range_of(ht, sizes->state);
    const Range inputs[] = {rq, rk, rv, rg, rb};
    for (const Range& r : inputs) {
        if (overlap(ro, r) || overlap(rht, r)) return GDR_ERR_ALIAS;
    }
    if (overlap(ro, rh0) || overlap(ro, rht)) return GDR_ERR_ALIAS;
    if (overlap(rht, rh0) && rht.lo != rh0.lo) return GDR_ERR_ALIAS;
    if (cu) {
        const Range rc = range_of(cu, ((size_t)d->B + 1) * 4);
        if (overlap(ro, rc) || overlap(rht, rc)) return GDR_ERR_ALIAS;
    }
    return GDR_OK;
}

gdr::LaunchArgs make_args(const gdr_dims* d, const void* q, const void* k, const void* v,
                          const void* g, const float* beta, const float* h0, void* o, float* ht,
                          void* workspace, void* stream, const int32_t* cu = nullptr) {
    gdr::LaunchArgs a{};
    a.B = d->B;
    a.T = d->T;
    a.HK = d->HK;
    a.HV = d->HV;
    a.dk = d->dk;
    a.dv = d->dv;
    a.chunk = d->chunk;
    a.qkv_f32 = d->qkv_dtype == GDR_F32;
    a.g_bf16 = (d->flags & GDR_G_BF16) != 0;
    a.k_l2norm = (d->flags & GDR_K_L2NORM) != 0;
    a.g_softplus = (d->flags & GDR_G_SOFTPLUS) != 0;
    a.o_bf16 = (d->flags & GDR_O_BF16) != 0;
    const bool gk = (d->flags & GDR_G_PER_KEY_HEAD) != 0;
    a.HG = gk ? d->HK : d->HV;
    const int G = d->HV / d->HK;
    if (d->flags & GDR_PREP_SPLIT)
        a.prep_split = true;
    else if (d->flags & GDR_PREP_FUSED)
        a.prep_split = false;
    else if (gk && G > 1 && G <= GDR_PREP_SPLIT_MAX_GROUP && d->chunk > 0) {
        // (batch element or sequence, key head, chunk) items of the prep
        const long long chunks = cu ? gdr::varlen_chunk_slots(d->B, d->T, d->chunk)
                                    : (long long)d->B * ((d->T + (long long)d->chunk - 1) / d->chunk);
        a.prep_split = gdr::split_prep_preferred(chunks * d->HK);
    }
    a.q = q;
    a.k = k;
    a.v = v;
    a.g = g;
    a.beta = beta;
    a.h0 = h0;
    a.o = o;
    a.ht = ht;
    a.workspace = workspace;
    a.stream = stream;
    a.cu_seqlens = cu;
    return a;
}

// Rows one prefill launch can address: the kernels reach one batch element's g/q/k/v/o rows
// (the padding rows of its last chunk included, which lie past the end and read as zero)
// and one head's chunk records with 31-bit buffer offsets.  The largest multiple of the
// chunk length W with (W + C) rows of HV heads x max(dk, dv) fp32 values and ceil(W / C)
// records each below 2^31 bytes (0 if not even one chunk fits).  Longer dense calls run as a
// chain of windows of W rows (see prefill_stages).
long long window_rows(const gdr_dims* d) {
    const long long C = d->chunk;
    const long long dmax = d->dk > d->dv ? d->dk : d->dv;
    const long long lim = (1LL << 31) - 1;
    long long w = lim / ((long long)d->HV * dmax * 4) - C;  // (w + C) rows < 2^31 bytes
    const gdr::ChunkRecord rec = gdr::ChunkRecord::make(d->chunk, d->dk);
    const long long wr = lim / rec.bytes * C;               // ceil(w / C) records < 2^31 bytes
    if (wr < w) w = wr;
    return w < C ? 0 : w / C * C;
}

size_t state_bytes(const gdr_dims* d) { return (size_t)d->HV * d->dk * d->dv * 4; }

// Whether T rows per batch element fit one launch: (T + C) rows of g and o and the records of
// ceil(T / C) chunks below 2^31 bytes (the padding rows of a ragged last chunk lie past the
// end but inside the range the offsets must cover).
bool fits_one_launch(const gdr_dims* d) {
    const size_t dmax = (size_t)(d->dk > d->dv ? d->dk : d->dv);
    const gdr::ChunkRecord rec = gdr::ChunkRecord::make(d->chunk, d->dk);
    const size_t nchunk = ((size_t)d->T + d->chunk - 1) / d->chunk;
    return ((size_t)d->T + d->chunk) * d->HV * dmax * 4 < (size_t(1) << 31) &&
           nchunk * (size_t)rec.bytes < (size_t(1) << 31);
}

size_t workspace_bytes_unchecked(const gdr_dims* d, bool varlen = false) {
    const gdr::ChunkRecord rec = gdr::ChunkRecord::make(d->chunk, d->dk);
    const long long W = window_rows(d);
    if (!varlen && W > 0 && !fits_one_launch(d)) {
        // a chain of windows of W rows, one batch element at a time: one window's records and
        // carry scratch, then one head group's state between windows
        size_t x;
        if (!mul_ok((size_t)d->HV, (size_t)(W / d->chunk), &x) || !mul_ok(x, rec.bytes, &x)) return 0;
        const size_t win = (gdr::carry_layout(1, d->HV, (int)W, d->dk, d->dv, d->chunk).total + 255) / 256 * 256;
        return win + state_bytes(d);
    }
    const size_t nchunk = varlen ? (size_t)gdr::varlen_chunk_slots(d->B, d->T, d->chunk)
                                 : (size_t)d->B * (((size_t)d->T + d->chunk - 1) / d->chunk);
    size_t x;
    if (!mul_ok((size_t)d->HV, nchunk, &x) || !mul_ok(x, rec.bytes, &x)) return 0;
    // the carry's segment summaries and start states (at most 256 heads x segments of
    // dk x dk fp32 matrices each), or a packed batch's plan, follow the records
    return gdr::carry_layout(d->B, d->HV, d->T, d->dk, d->dv, d->chunk, varlen).total;
}

bool prefill_dims_ok(const gdr_dims* dims) {
    return dims && dims->B >= 1 && dims->T >= 1 && dims->HK >= 1 && dims->HV >= 1 &&
           dims->HV % dims->HK == 0 && supported_head_dim(dims->dk) && supported_head_dim(dims->dv) &&
           (dims->chunk == 16 || dims->chunk == 32 || dims->chunk == 64);
}

}  // namespace

extern "C" {

int gdr_abi_version(void) { return GDR_ABI_VERSION; }

const char* gdr_status_str(int status) {
    switch (status) {
        case GDR_OK: return "ok";
        case GDR_ERR_NULL: return "a required pointer is NULL";
        case GDR_ERR_SHAPE: return "invalid shape (B/T/HK/HV, HV % HK, decode T != 1, or size overflow)";
        case GDR_ERR_UNSUPPORTED: return "unsupported head dim, chunk size or dtype";
        case GDR_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
        case GDR_ERR_ALIAS: return "output buffers overlap inputs, or ht partially overlaps h0";
        case GDR_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case GDR_ERR_HIP: return "HIP runtime error or kernel launch failure";
        case GDR_ERR_SCRATCH: return "call needs more workspace than the allocation-free entry point's scratch";
        default: return "unknown status";
    }
}

int gdr_decode_step(const gdr_dims* dims, const void* q, const void* k, const void* v,
                    const void* g, const float* beta, const float* h0, void* o, float* ht,
                    void* stream) {
    Sizes s;
    const int st = validate(dims, Path::decode, q, k, v, g, beta, h0, o, ht, &s);
    if (st != GDR_OK) return st;
    const gdr::LaunchArgs a = make_args(dims, q, k, v, g, beta, h0, o, ht, nullptr, stream);
    return gdr::launch_tokens(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int gdr_fused_recurrent(const gdr_dims* dims, const void* q, const void* k, const void* v,
                        const void* g, const float* beta, const float* h0, void* o, float* ht,
                        void* stream) {
    Sizes s;
    const int st = validate(dims, Path::tokens, q, k, v, g, beta, h0, o, ht, &s);
    if (st != GDR_OK) return st;
    const gdr::LaunchArgs a = make_args(dims, q, k, v, g, beta, h0, o, ht, nullptr, stream);
    return gdr::launch_tokens(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

size_t gdr_chunk_prefill_workspace_bytes(const gdr_dims* dims) {
    if (!prefill_dims_ok(dims)) return 0;
    return workspace_bytes_unchecked(dims);
}

size_t gdr_chunk_prefill_varlen_workspace_bytes(const gdr_dims* dims) {
    if (!prefill_dims_ok(dims) || dims->B > GDR_VARLEN_MAX_SEQS) return 0;
    return workspace_bytes_unchecked(dims, true);
}

// A dense prefill longer than W rows, as a chain of windows of W rows (a multiple of the chunk
// length, so the chunk grid is the one-call grid) per batch element: prep and carry of each
// window in order on the stream, the state handed from window to window through ht (in place)
// or, without ht, through a state slot after the window's records in the workspace.
static int prefill_windows(const gdr_dims* dims, long long W, const void* q, const void* k,
                           const void* v, const void* g, const float* beta, const float* h0,
                           void* o, float* ht, void* workspace, void* stream) {
    const size_t elt = dims->qkv_dtype == GDR_F32 ? 4 : 2;
    const size_t gelt = (dims->flags & GDR_G_BF16) ? 2 : 4;
    const size_t HG = (dims->flags & GDR_G_PER_KEY_HEAD) ? dims->HK : dims->HV;
    const size_t oelt = (dims->flags & GDR_O_BF16) ? 2 : 4;
    const size_t HK = dims->HK, HV = dims->HV, dk = dims->dk, dv = dims->dv;
    unsigned char* ws = static_cast<unsigned char*>(workspace);
    const size_t win = (gdr::carry_layout(1, dims->HV, (int)W, dims->dk, dims->dv, dims->chunk).total + 255) / 256 * 256;
    float* tmp = reinterpret_cast<float*>(ws + win);
    for (int b = 0; b < dims->B; ++b) {
        float* state = ht ? ht + (size_t)b * HV * dk * dv : tmp;
        for (long long t0 = 0; t0 < dims->T; t0 += W) {
            const long long t1 = t0 + W < dims->T ? t0 + W : dims->T;
            const size_t row = (size_t)b * dims->T + (size_t)t0;  // first row of the window
            gdr_dims dw = *dims;
            dw.B = 1;
            dw.T = (int32_t)(t1 - t0);
            const float* hin = t0 == 0 ? (h0 ? h0 + (size_t)b * HV * dk * dv : nullptr) : state;
            float* hout = (t1 == dims->T && !ht) ? nullptr : state;
            gdr::LaunchArgs a = make_args(&dw, static_cast<const unsigned char*>(q) + row * HK * dk * elt,
                                          static_cast<const unsigned char*>(k) + row * HK * dk * elt,
                                          static_cast<const unsigned char*>(v) + row * HV * dv * elt,
                                          static_cast<const unsigned char*>(g) + row * HG * dk * gelt,
                                          beta + row * HV, hin, static_cast<unsigned char*>(o) + row * HV * dv * oelt,
                                          hout, ws, stream);
            if (gdr::launch_chunk_prep(a) != hipSuccess || gdr::launch_chunk_carry(a) != hipSuccess)
                return GDR_ERR_HIP;
        }
    }
    return GDR_OK;
}

static int prefill_stages(const gdr_dims* dims, const void* q, const void* k, const void* v,
                          const void* g, const float* beta, const float* h0, void* o, float* ht,
                          void* workspace, size_t workspace_bytes, void* stream, bool prep,
                          bool carry, const int32_t* cu = nullptr) {
    Sizes s;
    const bool varlen = cu != nullptr;
    const int st = validate(dims, Path::chunked, q, k, v, g, beta, h0, o, ht, &s, cu, varlen);
    if (st != GDR_OK) return st;
    const size_t need = workspace_bytes_unchecked(dims, varlen);
    if (need == 0) return GDR_ERR_SHAPE;
    // Beyond the rows one launch can address (window_rows), a dense call runs as a chain of
    // windows; packed batches and the separate stage entry points do not chain.
    const long long W = window_rows(dims);
    const bool windowed = !fits_one_launch(dims);
    if (windowed && (W <= 0 || varlen || !prep || !carry)) return GDR_ERR_SHAPE;
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0 || workspace_bytes < need)
        return GDR_ERR_WORKSPACE;
    const Range rw = range_of(workspace, need);
    const Range others[] = {range_of(q, s.q), range_of(k, s.q), range_of(v, s.v), range_of(g, s.g),
                            range_of(beta, s.beta), range_of(h0, s.state), range_of(o, s.o),
                            range_of(ht, s.state), range_of(cu, ((size_t)dims->B + 1) * 4)};
    for (const Range& r : others)
        if (overlap(rw, r)) return GDR_ERR_ALIAS;
    if (windowed) return prefill_windows(dims, W, q, k, v, g, beta, h0, o, ht, workspace, stream);
    gdr::LaunchArgs a = make_args(dims, q, k, v, g, beta, h0, o, ht, workspace, stream, cu);
    if (varlen) {
        const gdr::CarryLayout L = gdr::carry_layout(dims->B, dims->HV, dims->T, dims->dk, dims->dv,
                                                     dims->chunk, true);
        a.plan = reinterpret_cast<int32_t*>(static_cast<unsigned char*>(workspace) + L.plan_off);
        a.nct = (int)gdr::varlen_chunk_slots(dims->B, dims->T, dims->chunk);
        if (prep && gdr::launch_varlen_plan(a) != hipSuccess) return GDR_ERR_HIP;
    }
    if (prep && gdr::launch_chunk_prep(a) != hipSuccess) return GDR_ERR_HIP;
    if (carry && gdr::launch_chunk_carry(a) != hipSuccess) return GDR_ERR_HIP;
    return GDR_OK;
}

int gdr_chunk_prefill(const gdr_dims* dims, const void* q, const void* k, const void* v,
                      const void* g, const float* beta, const float* h0, void* o, float* ht,
                      void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_stages(dims, q, k, v, g, beta, h0, o, ht, workspace, workspace_bytes, stream,
                          true, true);
}

int gdr_chunk_prefill_noalloc(const gdr_dims* dims, const void* q, const void* k, const void* v,
                              const void* g, const float* beta, const float* h0, void* o,
                              float* ht, void* stream) {
    Sizes s;
    const int st = validate(dims, Path::chunked, q, k, v, g, beta, h0, o, ht, &s);
    if (st != GDR_OK) return st;
    const size_t need = workspace_bytes_unchecked(dims);
    if (need == 0) return GDR_ERR_SHAPE;
    if (need > GDR_NOALLOC_SCRATCH_BYTES) return GDR_ERR_SCRATCH;
    void* ws = scratch_on_current_device();
    if (!ws) return GDR_ERR_HIP;
    return prefill_stages(dims, q, k, v, g, beta, h0, o, ht, ws, GDR_NOALLOC_SCRATCH_BYTES, stream,
                          true, true);
}

int gdr_chunk_prep(const gdr_dims* dims, const void* q, const void* k, const void* v,
                   const void* g, const float* beta, const float* h0, void* o, float* ht,
                   void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_stages(dims, q, k, v, g, beta, h0, o, ht, workspace, workspace_bytes, stream,
                          true, false);
}

int gdr_chunk_carry(const gdr_dims* dims, const void* q, const void* k, const void* v,
                    const void* g, const float* beta, const float* h0, void* o, float* ht,
                    void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_stages(dims, q, k, v, g, beta, h0, o, ht, workspace, workspace_bytes, stream,
                          false, true);
}

int gdr_chunk_prefill_varlen(const gdr_dims* dims, const int32_t* cu_seqlens, const void* q,
                             const void* k, const void* v, const void* g, const float* beta,
                             const float* h0, void* o, float* ht, void* workspace,
                             size_t workspace_bytes, void* stream) {
    if (!cu_seqlens) return GDR_ERR_NULL;
    return prefill_stages(dims, q, k, v, g, beta, h0, o, ht, workspace, workspace_bytes, stream,
                          true, true, cu_seqlens);
}

int gdr_fused_recurrent_varlen(const gdr_dims* dims, const int32_t* cu_seqlens, const void* q,
                               const void* k, const void* v, const void* g, const float* beta,
                               const float* h0, void* o, float* ht, void* stream) {
    Sizes s;
    const int st = validate(dims, Path::tokens, q, k, v, g, beta, h0, o, ht, &s, cu_seqlens, true);
    if (st != GDR_OK) return st;
    const gdr::LaunchArgs a = make_args(dims, q, k, v, g, beta, h0, o, ht, nullptr, stream, cu_seqlens);
    return gdr::launch_tokens(a) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int gdr_tree_verify(const gdr_dims* dims, const int32_t* parent, const void* q, const void* k,
                    const void* v, const void* g, const float* beta, const float* h0, void* o,
                    void* stream) {
    if (!parent) return GDR_ERR_NULL;
    Sizes s;
    const int st = validate(dims, Path::tokens, q, k, v, g, beta, h0, o, nullptr, &s);
    if (st != GDR_OK) return st;
    if (dims->T > GDR_TREE_MAX_T) return GDR_ERR_UNSUPPORTED;
    if ((reinterpret_cast<uintptr_t>(parent) & 3u) != 0) return GDR_ERR_ALIGN;
    if (overlap(range_of(o, s.o), range_of(parent, (size_t)dims->B * dims->T * 4))) return GDR_ERR_ALIAS;
    const gdr::LaunchArgs a = make_args(dims, q, k, v, g, beta, h0, o, nullptr, nullptr, stream);
    return gdr::launch_tree_verify(a, parent) == hipSuccess ? GDR_OK : GDR_ERR_HIP;
}

int gdr_forward(const gdr_dims* dims, const void* q, const void* k, const void* v,
                const void* g, const float* beta, const float* h0, void* o, float* ht,
                void* workspace, size_t workspace_bytes, void* stream) {
    if (dims && dims->T >= 1 && dims->T <= GDR_RECURRENT_MAX_T)
        return gdr_fused_recurrent(dims, q, k, v, g, beta, h0, o, ht, stream);
    return gdr_chunk_prefill(dims, q, k, v, g, beta, h0, o, ht, workspace, workspace_bytes, stream);
}

}  // extern "C"

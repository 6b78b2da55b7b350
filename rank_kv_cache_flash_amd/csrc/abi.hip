// abi.hip -- the C entry points declared in include/wsvd.h.
//
// Every check that the host can make happens here, before any HIP call, so
// a bad argument returns a negative status with nothing enqueued (and these
// paths work on a machine without a GPU).  Kernels live in decode.hip,
// combine.hip and append.hip.
#include <stdint.h>
#include <string.h>

#include <initializer_list>
#include <mutex>

#include "wsvd_common.hpp"
#include "wsvd_internal.hpp"

// Scratch of wsvd_decode_attn_noalloc, one copy per GPU for the life of the
// process: merge counters for up to kNoallocPairs (b, h) pairs in a region of
// their own (every call leaves them zero, so they never need clearing
// again), then the split partials (o_part, lse_part).  Host code never uses
// the name of this array as an address: each device's address comes from
// hipGetSymbolAddress (see noalloc_scratch below).
constexpr size_t kNoallocPairs = 65536;
constexpr size_t kNoallocCounterBytes = kNoallocPairs * sizeof(unsigned);   // 256 KiB
constexpr size_t kNoallocPartialBytes = size_t(16) << 20;                   // 16 MiB
static __device__ __align__(256) unsigned char scratch[kNoallocCounterBytes + kNoallocPartialBytes];

namespace {

// Automatic split choice, tuned on MI355X (256 CUs).  Each split block pays a
// fixed cost (both factors from L2, q' = B_K q, the projection and, with more
// than one split, the merge), so splits are only added where they buy
// parallelism: small batches get enough blocks to cover the CUs, large ones
// keep whole sequences per block and only cut long caches (which also evens
// out ragged lengths).
constexpr long kFillBlocks = 256;       // blocks wanted for a small batch
constexpr int kMinSplitTokens = 256;    // never cut sequences finer than this
constexpr int kLongTokens = 2048;       // large batches: caches up to this length stay whole
// Large batches with longer caches: splits of at most this many tokens
// (measured on MI355X, 64 sequences x 32 heads, 8192-token cache, ragged
// lengths: 5 or 6 splits 315.8-316.0 us per step, 4 splits 317.2-317.3, 8
// splits 317.8-317.9; cutting the 2048-token caches of the 32 x 32-head int8
// batch into 2 splits instead of 1 cost about 3 us).
constexpr int kLongSplitTokens = 1536;
constexpr long kLargeBatchPairs = 1024; // (b, h) pairs that make a batch "large"
// Split grids at least this large merge in a second launch (measured on
// MI355X: 8192 blocks gain 5.7 us from it, 160 blocks lose 1.35 us).
#ifndef WSVD_SEPARATE_MERGE_BLOCKS
#define WSVD_SEPARATE_MERGE_BLOCKS 2048
#endif
constexpr long kSeparateMergeBlocks = WSVD_SEPARATE_MERGE_BLOCKS;

// a * b * ... <= limit for non-negative factors, without overflowing (a
// product of several int sizes can pass 2^63).
bool product_le(std::initializer_list<long long> factors, long long limit) {
    long long p = 1;
    for (long long v : factors) {
        if (v < 0) return false;
        if (v == 0) return 0 <= limit;
        if (p > limit / v) return false;
        p *= v;
    }
    return p <= limit;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool act_dtype_ok(int dt) { return dt == WSVD_F32 || dt == WSVD_BF16 || dt == WSVD_F16; }
bool cache_dtype_ok(int dt) { return dt == WSVD_F32 || dt == WSVD_BF16 || dt == WSVD_I8; }
bool head_dim_ok(int H) { return H == 64 || H == 128; }
bool rank_ok(int r) { return r == 16 || r == 32 || r == 48 || r == 64; }
// The split kernel addresses one (b, h)'s rows with 32-bit byte offsets.
bool rows_fit(int L_cap, int row_elems, int dt) {
    const long long es = dt == WSVD_F32 ? 4 : dt == WSVD_I8 ? 1 : 2;
    return product_le({L_cap, row_elems, es}, (1ll << 31) - 1);
}

int resolve_splits(int nb, int nh, int L_cap, int n_splits) {
    if (nb <= 0 || nh <= 0 || L_cap <= 0 || n_splits < 0) return WSVD_ERR_SHAPE;
    if (n_splits > 0) return n_splits > L_cap ? WSVD_ERR_SHAPE : n_splits;
    const long bh = (long)nb * nh;
    long s = 1;
    if (bh < kFillBlocks) {
        s = (kFillBlocks + bh - 1) / bh;
        const long smax = ((long)L_cap + kMinSplitTokens - 1) / kMinSplitTokens;
        if (s > smax) s = smax;
    } else if (bh >= kLargeBatchPairs) {
        if (L_cap > kLongTokens) s = ((long)L_cap + kLongSplitTokens - 1) / kLongSplitTokens;
    }
    if (s < 1) s = 1;
    return (int)s;
}

size_t opart_bytes(int nb, int nh, int H, int S) { return (size_t)nb * nh * S * H * sizeof(float); }

// Large split grids merge in a second launch (see wsvd_decode_attn).
bool merge_separately(const wsvd::DecodeArgs& a) {
    return a.out != nullptr && a.S > 1 && (long)a.nb * a.nh * a.S >= kSeparateMergeBlocks;
}

template <class Launch>
int launch_with_merge(wsvd::DecodeArgs a, int H, Launch&& split, hipStream_t stream) {
    if (!merge_separately(a)) return split(a) == hipSuccess ? WSVD_OK : WSVD_ERR_HIP;
    void* out = a.out;
    a.out = nullptr;
    if (split(a) != hipSuccess) return WSVD_ERR_HIP;
    return wsvd::launch_combine(a.nb, a.nh, H, a.S, a.o_part, a.lse_part, out, a.out_dt, stream) == hipSuccess
               ? WSVD_OK
               : WSVD_ERR_HIP;
}

// Per-device address of `scratch`, looked up once per device with that
// device current; the first lookup also zero-fills the counter region on the
// caller's stream (device globals start zeroed, so this only makes the
// starting state explicit).
constexpr int kMaxDevices = 64;
struct ScratchSlot {
    std::once_flag once;
    void* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

hipError_t noalloc_scratch(hipStream_t stream, char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&] {
        void* p = nullptr;
        slot.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess)
            slot.err = wsvd::launch_fill_zero_u32(static_cast<unsigned*>(p), kNoallocPairs, stream);
        if (slot.err == hipSuccess) slot.ptr = p;
    });
    if (slot.err != hipSuccess) return slot.err;
    *out = static_cast<char*>(slot.ptr);
    return hipSuccess;
}

}  // namespace

extern "C" size_t wsvd_decode_counter_bytes(int nb, int nh);
extern "C" size_t wsvd_decode_opart_offset(int nb, int nh, int H, int L_cap, int n_splits);
extern "C" size_t wsvd_decode_lse_offset(int nb, int nh, int H, int L_cap, int n_splits);

namespace {

// Workspace layout: merge counters at byte 0 (nb * nh uint32, so their place
// does not depend on the split count), then o_part, then lse_part, each
// region 256-byte aligned.
void set_decode_workspace(wsvd::DecodeArgs& a, void* workspace, int nb, int nh, int H, int L_cap, int n_splits) {
    char* ws = static_cast<char*>(workspace);
    a.counters = reinterpret_cast<unsigned*>(ws);
    a.o_part = reinterpret_cast<float*>(ws + wsvd_decode_opart_offset(nb, nh, H, L_cap, n_splits));
    a.lse_part = reinterpret_cast<float*>(ws + wsvd_decode_lse_offset(nb, nh, H, L_cap, n_splits));
}

}  // namespace

extern "C" {

int wsvd_decode_num_splits(int nb, int nh, int L_cap, int n_splits) {
    return resolve_splits(nb, nh, L_cap, n_splits);
}

size_t wsvd_decode_counter_bytes(int nb, int nh) {
    if (nb <= 0 || nh <= 0) return 0;
    return round_up((size_t)nb * nh * sizeof(unsigned), 256);
}

size_t wsvd_decode_opart_offset(int nb, int nh, int H, int L_cap, int n_splits) {
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0 || H <= 0) return 0;
    return wsvd_decode_counter_bytes(nb, nh);
}

size_t wsvd_decode_lse_offset(int nb, int nh, int H, int L_cap, int n_splits) {
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0 || H <= 0) return 0;
    return wsvd_decode_counter_bytes(nb, nh) + round_up(opart_bytes(nb, nh, H, S), 256);
}

size_t wsvd_decode_workspace_bytes(int nb, int nh, int H, int L_cap, int n_splits) {
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0 || H <= 0) return 0;
    return wsvd_decode_lse_offset(nb, nh, H, L_cap, n_splits) + round_up((size_t)nb * nh * S * sizeof(float), 256);
}

// One append workspace serves both forms of the call at these sizes: the
// bf16-operand kernel and the int8-operand kernel.
size_t wsvd_append_counter_bytes(int nb, int nh, int r) {
    if (nb <= 0 || nh <= 0 || r <= 0) return 0;
    const int NT = wsvd::append_bf16_tile_cols(WSVD_BF16, r);
    long tiles = wsvd::append_w8_num_tiles(nb, nh, r);
    const long t = wsvd::append_bf16_num_tiles(nb, nh, r, NT);
    if (t > tiles) tiles = t;
    return round_up((size_t)tiles * sizeof(unsigned), 256);
}

size_t wsvd_append_workspace_bytes(int nb, int E, int nh, int r) {
    if (nb <= 0 || E <= 0 || nh <= 0 || r <= 0) return 0;
    const int NT = wsvd::append_bf16_tile_cols(WSVD_BF16, r);
    size_t part = wsvd::append_w8_partial_bytes(nb, E, nh, r);
    const size_t p = wsvd::append_bf16_partial_bytes(nb, E, nh, r, NT);
    if (p > part) part = p;
    if (part == 0) return 0;
    return wsvd_append_counter_bytes(nb, nh, r) + round_up(part, 256);
}

const char* wsvd_status_string(int st) {
    switch (st) {
        case WSVD_OK: return "ok";
        case WSVD_ERR_NULL: return "a required pointer is NULL";
        case WSVD_ERR_SHAPE: return "invalid or inconsistent sizes";
        case WSVD_ERR_DTYPE: return "dtype not allowed for this argument";
        case WSVD_ERR_UNSUPPORTED: return "shape/dtype combination not compiled";
        case WSVD_ERR_ALIGN: return "pointer not 16-byte aligned";
        case WSVD_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case WSVD_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

const char* wsvd_version(void) { return "wsvd 0.1 gfx950"; }

// Host checks of wsvd_decode_attn except the workspace; on success fills
// everything in `a` but the workspace pointers.
static int check_decode(int nb, int nh, int H, int r, int L_cap, const int32_t* L, const void* q, wsvd_dtype q_dt,
                        const void* C_K, const void* C_V, wsvd_dtype C_dt, const uint16_t* s_K, const uint16_t* s_V,
                        const void* B_K, const void* B_V, wsvd_dtype B_dt, float softmax_scale, int n_splits,
                        void* out, wsvd_dtype out_dt, wsvd::DecodeArgs& a) {
    if (nb <= 0 || nh <= 0 || H <= 0 || r <= 0 || L_cap <= 0 || n_splits < 0 || r > H) return WSVD_ERR_SHAPE;
    if (!product_le({nb, nh, L_cap, r}, 1ll << 46)) return WSVD_ERR_SHAPE;
    if (!L || !q || !C_K || !C_V || !B_K || !B_V) return WSVD_ERR_NULL;
    if (!act_dtype_ok(q_dt) || !act_dtype_ok(B_dt) || !cache_dtype_ok(C_dt)) return WSVD_ERR_DTYPE;
    if (out && !act_dtype_ok(out_dt)) return WSVD_ERR_DTYPE;
    if (C_dt == WSVD_I8 && (!s_K || !s_V)) return WSVD_ERR_NULL;
    if (!rows_fit(L_cap, r, C_dt)) return WSVD_ERR_SHAPE;
    if (!head_dim_ok(H) || !rank_ok(r)) return WSVD_ERR_UNSUPPORTED;
    if (!aligned16(L) || !aligned16(q) || !aligned16(C_K) || !aligned16(C_V) || !aligned16(B_K) ||
        !aligned16(B_V) || (out && !aligned16(out)))
        return WSVD_ERR_ALIGN;
    if (C_dt == WSVD_I8 && (!aligned16(s_K) || !aligned16(s_V))) return WSVD_ERR_ALIGN;
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0) return WSVD_ERR_SHAPE;
    if (!product_le({nb, nh, S}, (1ll << 31) - 1)) return WSVD_ERR_SHAPE;

    memset(&a, 0, sizeof(a));
    a.nb = nb;
    a.nh = nh;
    a.L_cap = L_cap;
    a.S = S;
    a.L = L;
    a.q = q;
    a.q_dt = q_dt;
    a.C_K = C_K;
    a.C_V = C_V;
    a.s_K = C_dt == WSVD_I8 ? s_K : nullptr;
    a.s_V = C_dt == WSVD_I8 ? s_V : nullptr;
    a.B_K = B_K;
    a.B_V = B_V;
    a.B_dt = B_dt;
    const float sigma = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)H);
    a.scale_log2 = sigma * wsvd::kLog2e;
    a.out = out;
    a.out_dt = out ? (int)out_dt : 0;
    return WSVD_OK;
}

int wsvd_decode_attn(int nb, int nh, int H, int r, int L_cap, const int32_t* L, const void* q, wsvd_dtype q_dt,
                     const void* C_K, const void* C_V, wsvd_dtype C_dt, const uint16_t* s_K, const uint16_t* s_V,
                     const void* B_K, const void* B_V, wsvd_dtype B_dt, float softmax_scale, int n_splits,
                     void* workspace, size_t workspace_bytes, void* out, wsvd_dtype out_dt, hipStream_t stream) {
    wsvd::DecodeArgs a;
    const int st = check_decode(nb, nh, H, r, L_cap, L, q, q_dt, C_K, C_V, C_dt, s_K, s_V, B_K, B_V, B_dt,
                                softmax_scale, n_splits, out, out_dt, a);
    if (st != WSVD_OK) return st;
    const size_t need = wsvd_decode_workspace_bytes(nb, nh, H, L_cap, n_splits);
    if (!workspace || !aligned256(workspace) || workspace_bytes < need) return WSVD_ERR_WORKSPACE;
    set_decode_workspace(a, workspace, nb, nh, H, L_cap, n_splits);

    // With out and S > 1: on a grid that is resident in about two rounds the
    // last split of each head merges (one launch); on larger grids every
    // block would otherwise hold its slot through the store-and-arrive round
    // trip, so the splits write partials only and the merge kernel follows.
    return launch_with_merge(
        a, H, [&](const wsvd::DecodeArgs& x) { return wsvd::launch_decode_split(x, H, r, C_dt, stream); }, stream);
}

int wsvd_decode_attn_noalloc(int nb, int nh, int H, int r, int L_cap, const int32_t* L, const void* q,
                             wsvd_dtype q_dt, const void* C_K, const void* C_V, wsvd_dtype C_dt, const uint16_t* s_K,
                             const uint16_t* s_V, const void* B_K, const void* B_V, wsvd_dtype B_dt,
                             float softmax_scale, int n_splits, void* out, wsvd_dtype out_dt, hipStream_t stream) {
    if (!out) return WSVD_ERR_NULL;  // the partials stay in the library's scratch: only out is a result
    wsvd::DecodeArgs a;
    const int st = check_decode(nb, nh, H, r, L_cap, L, q, q_dt, C_K, C_V, C_dt, s_K, s_V, B_K, B_V, B_dt,
                                softmax_scale, n_splits, out, out_dt, a);
    if (st != WSVD_OK) return st;
    // The partial regions laid out as in a caller workspace, after the fixed
    // counter region; sizes beyond the scratch are refused.
    const size_t part = wsvd_decode_workspace_bytes(nb, nh, H, L_cap, n_splits) - wsvd_decode_counter_bytes(nb, nh);
    if ((size_t)nb * nh > kNoallocPairs || part > kNoallocPartialBytes) return WSVD_ERR_WORKSPACE;
    char* base = nullptr;
    if (noalloc_scratch(stream, &base) != hipSuccess) return WSVD_ERR_HIP;
    const size_t ctr = wsvd_decode_counter_bytes(nb, nh);
    a.counters = reinterpret_cast<unsigned*>(base);
    a.o_part = reinterpret_cast<float*>(base + kNoallocCounterBytes +
                                        (wsvd_decode_opart_offset(nb, nh, H, L_cap, n_splits) - ctr));
    a.lse_part = reinterpret_cast<float*>(base + kNoallocCounterBytes +
                                          (wsvd_decode_lse_offset(nb, nh, H, L_cap, n_splits) - ctr));
    return launch_with_merge(
        a, H, [&](const wsvd::DecodeArgs& x) { return wsvd::launch_decode_split(x, H, r, C_dt, stream); }, stream);
}

int wsvd_dense_decode_attn(int nb, int nh, int H, int L_cap, const int32_t* L, const void* q, wsvd_dtype q_dt,
                           const void* K, const void* V, wsvd_dtype kv_dt, float softmax_scale, int n_splits,
                           void* workspace, size_t workspace_bytes, void* out, wsvd_dtype out_dt,
                           hipStream_t stream) {
    if (nb <= 0 || nh <= 0 || H <= 0 || L_cap <= 0 || n_splits < 0) return WSVD_ERR_SHAPE;
    if (!product_le({nb, nh, L_cap, H}, 1ll << 46)) return WSVD_ERR_SHAPE;
    if (!L || !q || !K || !V) return WSVD_ERR_NULL;
    if (!act_dtype_ok(q_dt) || kv_dt != WSVD_BF16) return WSVD_ERR_DTYPE;
    if (out && !act_dtype_ok(out_dt)) return WSVD_ERR_DTYPE;
    if (!rows_fit(L_cap, H, kv_dt)) return WSVD_ERR_SHAPE;
    if (!head_dim_ok(H)) return WSVD_ERR_UNSUPPORTED;
    if (!aligned16(L) || !aligned16(q) || !aligned16(K) || !aligned16(V) || (out && !aligned16(out)))
        return WSVD_ERR_ALIGN;
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0) return WSVD_ERR_SHAPE;
    if (!product_le({nb, nh, S}, (1ll << 31) - 1)) return WSVD_ERR_SHAPE;
    const size_t need = wsvd_decode_workspace_bytes(nb, nh, H, L_cap, n_splits);
    if (!workspace || !aligned256(workspace) || workspace_bytes < need) return WSVD_ERR_WORKSPACE;

    wsvd::DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.nb = nb;
    a.nh = nh;
    a.L_cap = L_cap;
    a.S = S;
    a.L = L;
    a.q = q;
    a.q_dt = q_dt;
    a.C_K = K;
    a.C_V = V;
    a.B_dt = WSVD_BF16;
    const float sigma = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)H);
    a.scale_log2 = sigma * wsvd::kLog2e;
    set_decode_workspace(a, workspace, nb, nh, H, L_cap, n_splits);
    a.out = out;
    a.out_dt = out ? (int)out_dt : 0;
    return launch_with_merge(
        a, H, [&](const wsvd::DecodeArgs& x) { return wsvd::launch_dense_split(x, H, stream); }, stream);
}

int wsvd_rope_tables(int L_cap, int H, float base, float* rope_cos, float* rope_sin, hipStream_t stream) {
    if (L_cap <= 0 || H <= 0 || H % 2 != 0 || !(base > 1.0f)) return WSVD_ERR_SHAPE;
    if (!rope_cos || !rope_sin) return WSVD_ERR_NULL;
    if ((long long)L_cap * H > (1ll << 40)) return WSVD_ERR_SHAPE;
    if (!aligned16(rope_cos) || !aligned16(rope_sin)) return WSVD_ERR_ALIGN;
    return wsvd::launch_rope_tables(L_cap, H, (double)base, rope_cos, rope_sin, stream) == hipSuccess ? WSVD_OK
                                                                                                      : WSVD_ERR_HIP;
}

int wsvd_decode_attn_rope(int nb, int nh, int H, int r, int L_cap, const int32_t* L, const void* q,
                          wsvd_dtype q_dt, const void* C_K, const void* C_V, wsvd_dtype C_dt, const void* B_K,
                          const void* B_V, wsvd_dtype B_dt, const float* rope_cos, const float* rope_sin,
                          float softmax_scale, int n_splits, void* workspace, size_t workspace_bytes, void* out,
                          wsvd_dtype out_dt, hipStream_t stream) {
    if (nb <= 0 || nh <= 0 || H <= 0 || r <= 0 || L_cap <= 0 || n_splits < 0 || r > H) return WSVD_ERR_SHAPE;
    if (!product_le({nb, nh, L_cap, r}, 1ll << 46)) return WSVD_ERR_SHAPE;
    if (!L || !q || !C_K || !C_V || !B_K || !B_V || !rope_cos || !rope_sin) return WSVD_ERR_NULL;
    if (!act_dtype_ok(q_dt) || B_dt != WSVD_BF16 || C_dt != WSVD_BF16) return WSVD_ERR_DTYPE;
    if (out && !act_dtype_ok(out_dt)) return WSVD_ERR_DTYPE;
    if (!head_dim_ok(H) || (r != 32 && r != 64)) return WSVD_ERR_UNSUPPORTED;
    if (!aligned16(L) || !aligned16(q) || !aligned16(C_K) || !aligned16(C_V) || !aligned16(B_K) ||
        !aligned16(B_V) || !aligned16(rope_cos) || !aligned16(rope_sin) || (out && !aligned16(out)))
        return WSVD_ERR_ALIGN;
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0) return WSVD_ERR_SHAPE;
    if (!product_le({nb, nh, S}, (1ll << 31) - 1)) return WSVD_ERR_SHAPE;
    const size_t need = wsvd_decode_workspace_bytes(nb, nh, H, L_cap, n_splits);
    if (!workspace || !aligned256(workspace) || workspace_bytes < need) return WSVD_ERR_WORKSPACE;

    wsvd::DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.nb = nb;
    a.nh = nh;
    a.L_cap = L_cap;
    a.S = S;
    a.L = L;
    a.q = q;
    a.q_dt = q_dt;
    a.C_K = C_K;
    a.C_V = C_V;
    a.B_K = B_K;
    a.B_V = B_V;
    a.B_dt = B_dt;
    const float sigma = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)H);
    a.scale_log2 = sigma * wsvd::kLog2e;
    set_decode_workspace(a, workspace, nb, nh, H, L_cap, n_splits);
    a.out = out;
    a.out_dt = out ? (int)out_dt : 0;
    return launch_with_merge(
        a, H, [&](const wsvd::DecodeArgs& x) { return wsvd::launch_decode_rope(x, H, r, rope_cos, rope_sin, stream); },
        stream);
}

int wsvd_combine_splits(int nb, int nh, int H, int n_splits, const float* o_part, const float* lse_part, void* out,
                        wsvd_dtype out_dt, hipStream_t stream) {
    if (nb <= 0 || nh <= 0 || H <= 0 || n_splits <= 0) return WSVD_ERR_SHAPE;
    if (!o_part || !lse_part || !out) return WSVD_ERR_NULL;
    if (!act_dtype_ok(out_dt)) return WSVD_ERR_DTYPE;
    if (!head_dim_ok(H)) return WSVD_ERR_UNSUPPORTED;
    if (!aligned16(o_part) || !aligned16(lse_part) || !aligned16(out)) return WSVD_ERR_ALIGN;
    if ((long long)nb * nh >= (1ll << 31)) return WSVD_ERR_SHAPE;
    return wsvd::launch_combine(nb, nh, H, n_splits, o_part, lse_part, out, out_dt, stream) == hipSuccess
               ? WSVD_OK
               : WSVD_ERR_HIP;
}

static bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

int wsvd_w8a8_quantize_activations(int nb, int E, const void* x, wsvd_dtype x_dt, int8_t* xq, float* sx,
                                   hipStream_t stream) {
    if (nb <= 0 || E <= 0) return WSVD_ERR_SHAPE;
    if (!x || !xq || !sx) return WSVD_ERR_NULL;
    if (!act_dtype_ok(x_dt)) return WSVD_ERR_DTYPE;
    if (!pow2_in(E, 256, 8192)) return WSVD_ERR_UNSUPPORTED;
    if ((long long)nb * E > (1ll << 40)) return WSVD_ERR_SHAPE;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(sx)) return WSVD_ERR_ALIGN;
    return wsvd::launch_w8a8_quantize_rows(nb, E, x, x_dt, xq, sx, stream) == hipSuccess ? WSVD_OK : WSVD_ERR_HIP;
}

int wsvd_w8a8_prepare_factor(int E, int N, const void* A, wsvd_dtype A_dt, int8_t* AqT, float* sA,
                             hipStream_t stream) {
    if (E <= 0 || N <= 0) return WSVD_ERR_SHAPE;
    if (!A || !AqT || !sA) return WSVD_ERR_NULL;
    if (!act_dtype_ok(A_dt)) return WSVD_ERR_DTYPE;
    if (!pow2_in(E, 256, 8192)) return WSVD_ERR_UNSUPPORTED;
    if ((long long)E * N > (1ll << 40)) return WSVD_ERR_SHAPE;
    if (!aligned16(A) || !aligned16(AqT) || !aligned16(sA)) return WSVD_ERR_ALIGN;
    return wsvd::launch_w8a8_prepare(E, N, A, A_dt, AqT, sA, stream) == hipSuccess ? WSVD_OK : WSVD_ERR_HIP;
}

// Checks shared by both append entry points (everything but the operands).
static int check_append_common(int nb, int E, int nh, int r, int L_cap, const int32_t* pos, void* C_K, void* C_V,
                               wsvd_dtype C_dt, uint16_t* s_K, uint16_t* s_V, void* workspace,
                               size_t workspace_bytes, int e_multiple) {
    if (!pos || !C_K || !C_V) return WSVD_ERR_NULL;
    if (!cache_dtype_ok(C_dt)) return WSVD_ERR_DTYPE;
    if (C_dt == WSVD_I8) {
        if (!s_K || !s_V) return WSVD_ERR_NULL;
        if (!aligned16(s_K) || !aligned16(s_V)) return WSVD_ERR_ALIGN;
        if (r == 48) return WSVD_ERR_UNSUPPORTED;  // a head must be whole 16-column groups of one 64-column tile
    } else if (s_K || s_V) {
        return WSVD_ERR_SHAPE;
    }
    if (!rank_ok(r) || E % e_multiple != 0) return WSVD_ERR_UNSUPPORTED;
    if (!product_le({nb, nh, L_cap, r}, 1ll << 46) || !product_le({E, nh, r}, 1ll << 30) ||
        !product_le({nb, E}, 1ll << 30))
        return WSVD_ERR_SHAPE;
    if (!aligned16(pos) || !aligned16(C_K) || !aligned16(C_V)) return WSVD_ERR_ALIGN;
    const size_t need = wsvd_append_workspace_bytes(nb, E, nh, r);
    if (need > 0 && (!workspace || !aligned256(workspace) || workspace_bytes < need)) return WSVD_ERR_WORKSPACE;
    return WSVD_OK;
}

static wsvd::AppendArgs append_args(int nb, int E, int nh, int r, int L_cap, const int32_t* pos, void* C_K,
                                    void* C_V, wsvd_dtype C_dt, uint16_t* s_K, uint16_t* s_V, void* workspace) {
    wsvd::AppendArgs a{};
    a.nb = nb;
    a.E = E;
    a.nh = nh;
    a.r = r;
    a.L_cap = L_cap;
    a.pos = pos;
    a.C_K = C_K;
    a.C_V = C_V;
    a.C_dt = C_dt;
    a.s_K = s_K;
    a.s_V = s_V;
    // Counters at byte 0 (one per output tile), then the partial tiles.
    const size_t need = wsvd_append_workspace_bytes(nb, E, nh, r);
    a.counters = need > 0 ? static_cast<unsigned*>(workspace) : nullptr;
    a.part = need > 0 ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                                 wsvd_append_counter_bytes(nb, nh, r))
                      : nullptr;
    return a;
}

int wsvd_append_latent_w8a8(int nb, int E, int nh, int r, int L_cap, const int8_t* xq, const float* sx,
                            const int8_t* AqT_K, const int8_t* AqT_V, const float* sA_K, const float* sA_V,
                            const int32_t* pos, void* C_K, void* C_V, wsvd_dtype C_dt, uint16_t* s_K,
                            uint16_t* s_V, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (nb <= 0 || E <= 0 || nh <= 0 || r <= 0 || L_cap <= 0) return WSVD_ERR_SHAPE;
    if (!xq || !sx || !AqT_K || !AqT_V || !sA_K || !sA_V) return WSVD_ERR_NULL;
    if (!aligned16(xq) || !aligned16(sx) || !aligned16(AqT_K) || !aligned16(AqT_V) || !aligned16(sA_K) ||
        !aligned16(sA_V))
        return WSVD_ERR_ALIGN;
    const int st = check_append_common(nb, E, nh, r, L_cap, pos, C_K, C_V, C_dt, s_K, s_V, workspace,
                                       workspace_bytes, 512);
    if (st != WSVD_OK) return st;
    wsvd::AppendArgs a = append_args(nb, E, nh, r, L_cap, pos, C_K, C_V, C_dt, s_K, s_V, workspace);
    a.KS = wsvd::append_w8_num_esplits(nb, E, nh, r);
    a.w8 = 1;
    a.x = xq;
    a.sx = sx;
    a.A_K = AqT_K;
    a.A_V = AqT_V;
    a.sA_K = sA_K;
    a.sA_V = sA_V;
    return wsvd::launch_append_w8(a, stream) == hipSuccess ? WSVD_OK : WSVD_ERR_HIP;
}

int wsvd_append_latent(int nb, int E, int nh, int r, int L_cap, const void* x, wsvd_dtype x_dt, const void* A_K,
                       const void* A_V, wsvd_dtype A_dt, const int32_t* pos, void* C_K, void* C_V, wsvd_dtype C_dt,
                       uint16_t* s_K, uint16_t* s_V, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (nb <= 0 || E <= 0 || nh <= 0 || r <= 0 || L_cap <= 0) return WSVD_ERR_SHAPE;
    if (!x || !A_K || !A_V) return WSVD_ERR_NULL;
    if (x_dt != WSVD_BF16 || A_dt != WSVD_BF16) return WSVD_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(A_K) || !aligned16(A_V)) return WSVD_ERR_ALIGN;
    const int st = check_append_common(nb, E, nh, r, L_cap, pos, C_K, C_V, C_dt, s_K, s_V, workspace,
                                       workspace_bytes, 256);
    if (st != WSVD_OK) return st;
    wsvd::AppendArgs a = append_args(nb, E, nh, r, L_cap, pos, C_K, C_V, C_dt, s_K, s_V, workspace);
    a.w8 = 0;
    a.KS = wsvd::append_bf16_num_esplits(nb, E, nh, r, wsvd::append_bf16_tile_cols(C_dt, r));
    a.x = x;
    a.A_K = A_K;
    a.A_V = A_V;
    return wsvd::launch_append_bf16(a, stream) == hipSuccess ? WSVD_OK : WSVD_ERR_HIP;
}

int wsvd_floor_probe(int mode, int blocks, const void* src, size_t bytes, float* sink, hipStream_t stream) {
    if ((mode != 0 && mode != 1) || blocks <= 0 || blocks > (1 << 20)) return WSVD_ERR_SHAPE;
    if (!sink || (mode == 1 && !src)) return WSVD_ERR_NULL;
    if (!aligned16(sink) || (mode == 1 && !aligned16(src))) return WSVD_ERR_ALIGN;
    // mode 1: at most 16 loads of 16 bytes per thread, whole 16-byte chunks per block
    if (mode == 1 && (bytes == 0 || bytes % (16 * (size_t)blocks) != 0 || bytes / 16 / (size_t)blocks > 16 * 256))
        return WSVD_ERR_SHAPE;
    return wsvd::launch_probe(mode, blocks, src, bytes, sink, stream) == hipSuccess ? WSVD_OK : WSVD_ERR_HIP;
}

size_t wsvd_factorize_svd_workspace_bytes(int E, int nh, int H) {
    if (E <= 0 || nh <= 0 || !head_dim_ok(H)) return 0;
    return (size_t)wsvd::svd_num_chunks(E, nh) * nh * H * H * sizeof(double);
}

int wsvd_factorize_svd(int E, int nh, int H, int r, const float* W, float* A, float* B, float* sigma, int* sweeps,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (E <= 0 || nh <= 0 || r <= 0 || H <= 0 || r > H) return WSVD_ERR_SHAPE;
    if (nh > 65535 || !product_le({E, nh, H}, 1ll << 40)) return WSVD_ERR_SHAPE;
    if (!head_dim_ok(H)) return WSVD_ERR_UNSUPPORTED;
    if (!W || !A || !B || !sigma) return WSVD_ERR_NULL;
    if (!aligned16(W) || !aligned16(A) || !aligned16(B) || !aligned16(sigma)) return WSVD_ERR_ALIGN;
    const size_t need = wsvd_factorize_svd_workspace_bytes(E, nh, H);
    if (!workspace || !aligned16(workspace) || workspace_bytes < need) return WSVD_ERR_WORKSPACE;
    return wsvd::launch_factorize_svd(W, E, nh, H, r, A, B, sigma, sweeps, static_cast<double*>(workspace), stream) ==
                   hipSuccess
               ? WSVD_OK
               : WSVD_ERR_HIP;
}

static int check_weighted(int E, int nh, int H, int r, const float* W, const float* F, const float* in,
                          const float* out) {
    if (E <= 0 || nh <= 0 || r <= 0 || H <= 0 || r > H) return WSVD_ERR_SHAPE;
    if (nh > 65535 || !product_le({E, nh, H}, 1ll << 40)) return WSVD_ERR_SHAPE;
    if (!head_dim_ok(H) || !rank_ok(r)) return WSVD_ERR_UNSUPPORTED;
    if (!W || !F || !in || !out) return WSVD_ERR_NULL;
    if (!aligned16(W) || !aligned16(F) || !aligned16(in) || !aligned16(out)) return WSVD_ERR_ALIGN;
    return WSVD_OK;
}

int wsvd_weighted_update_A(int E, int nh, int H, int r, const float* W, const float* F, const float* B, float* A,
                           hipStream_t stream) {
    const int st = check_weighted(E, nh, H, r, W, F, B, A);
    if (st != WSVD_OK) return st;
    return wsvd::launch_factorize_weighted(true, W, F, B, E, nh, H, r, A, stream) == hipSuccess ? WSVD_OK
                                                                                               : WSVD_ERR_HIP;
}

int wsvd_weighted_update_B(int E, int nh, int H, int r, const float* W, const float* F, const float* A, float* B,
                           hipStream_t stream) {
    const int st = check_weighted(E, nh, H, r, W, F, A, B);
    if (st != WSVD_OK) return st;
    return wsvd::launch_factorize_weighted(false, W, F, A, E, nh, H, r, B, stream) == hipSuccess ? WSVD_OK
                                                                                                : WSVD_ERR_HIP;
}

static size_t shared_qp_bytes(int nb, int nh, int R) { return round_up((size_t)nb * nh * R * sizeof(float), 256); }
static size_t shared_part_bytes(int nb, int nh, int R, int S) {
    return round_up((size_t)nb * nh * S * R * sizeof(float), 256);
}

// fp32 [R / 128, nb, nh, H] chunk contributions of the projection (H <= 128).
static size_t shared_proj_bytes(int nb, int nh, int R) {
    return round_up((size_t)((R + 127) / 128) * nb * nh * 128 * sizeof(float), 256);
}

size_t wsvd_shared_decode_workspace_bytes(int nb, int nh, int R, int L_cap, int n_splits) {
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0 || R <= 0) return 0;
    return shared_qp_bytes(nb, nh, R) + shared_part_bytes(nb, nh, R, S) +
           round_up((size_t)nb * nh * S * sizeof(float), 256) + shared_proj_bytes(nb, nh, R);
}

int wsvd_shared_decode_attn(int nb, int nh, int H, int R, int L_cap, const int32_t* L, const void* q,
                            const void* C_K, const void* C_V, const void* B_K, const void* B_V, float softmax_scale,
                            int n_splits, void* workspace, size_t workspace_bytes, void* out, wsvd_dtype out_dt,
                            hipStream_t stream) {
    if (nb <= 0 || nh <= 0 || H <= 0 || R <= 0 || L_cap <= 0 || n_splits < 0) return WSVD_ERR_SHAPE;
    if (nh > 4096 || !product_le({nb, L_cap, R}, 1ll << 40) || !product_le({R, nh, H}, 1ll << 40))
        return WSVD_ERR_SHAPE;
    if (!L || !q || !C_K || !C_V || !B_K || !B_V || !out) return WSVD_ERR_NULL;
    if (out_dt != WSVD_F32 && out_dt != WSVD_BF16) return WSVD_ERR_DTYPE;
    if (!head_dim_ok(H) || (R != 512 && R != 1024 && R != 2048)) return WSVD_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(C_K) || !aligned16(C_V) || !aligned16(B_K) || !aligned16(B_V) ||
        !aligned16(out) || !aligned16(L))
        return WSVD_ERR_ALIGN;
    const int S = resolve_splits(nb, nh, L_cap, n_splits);
    if (S <= 0) return WSVD_ERR_SHAPE;
    if (!product_le({nb, S, nh}, (1ll << 31) - 4096)) return WSVD_ERR_SHAPE;
    const size_t need = wsvd_shared_decode_workspace_bytes(nb, nh, R, L_cap, n_splits);
    if (!workspace || !aligned256(workspace) || workspace_bytes < need) return WSVD_ERR_WORKSPACE;
    wsvd::SharedArgs a;
    a.nb = nb;
    a.nh = nh;
    a.H = H;
    a.R = R;
    a.L_cap = L_cap;
    a.S = S;
    a.L = L;
    a.q = static_cast<const uint16_t*>(q);
    a.C_K = static_cast<const uint16_t*>(C_K);
    a.C_V = static_cast<const uint16_t*>(C_V);
    a.B_K = static_cast<const uint16_t*>(B_K);
    a.B_V = static_cast<const uint16_t*>(B_V);
    const float sigma = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)H);
    a.scale_log2 = sigma * wsvd::kLog2e;
    char* ws = static_cast<char*>(workspace);
    a.qp = reinterpret_cast<float*>(ws);
    a.o_part = reinterpret_cast<float*>(ws + shared_qp_bytes(nb, nh, R));
    a.lse_part = reinterpret_cast<float*>(ws + shared_qp_bytes(nb, nh, R) + shared_part_bytes(nb, nh, R, S));
    a.proj_part = reinterpret_cast<float*>(ws + shared_qp_bytes(nb, nh, R) + shared_part_bytes(nb, nh, R, S) +
                                           round_up((size_t)nb * nh * S * sizeof(float), 256));
    a.out = out;
    a.out_dt = (int)out_dt;
    return wsvd::launch_shared_decode(a, stream) == hipSuccess ? WSVD_OK : WSVD_ERR_HIP;
}

}  // extern "C"


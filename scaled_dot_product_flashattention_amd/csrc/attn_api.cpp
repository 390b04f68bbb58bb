// C ABI of libattn (declared in include/attn.h): argument validation, the
// choice between the fused kernel and the split-over-keys pair, and launch.
// Every check runs on the host before any HIP call, so a rejected call never
// touches the GPU.
#include "attn.h"

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>

#include "launch.h"

namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
// Split plan for one query over many keys (measured on MI355X over decode
// shapes of 8 to 1024 heads and 4096 to 131072 keys): the split kernels beat
// the fused kernel for a single query per head (its 128-query tiles would be
// almost empty), and run best with about 2 workgroups per compute unit and
// at most about 4096 keys per split. They stream K and V once per query row,
// so from two queries per head on, the fused kernel, which reads them once
// per query tile, is faster (4 queries: 2441 us split against 764 us fused
// at B8 H32 Sk32768).
constexpr int kSplitMaxQueries = 1;      // query rows per head at which the split path is used
constexpr int kSplitTargetGroups = 512;  // about 2 workgroups per compute unit
constexpr int kSplitMaxKeys = 4096;      // keys per split, at most (more splits past that)
constexpr int kSplitMinKeys = 512;       // keys per split, at least
// Key splits of the fused 16-bit kernel, for two or more queries per head:
// when its (batch, head, 128-query tile) workgroups would not fill the
// compute units and the keys are long, each workgroup takes one key range
// and the merge kernel combines the ranges' records. The ranges run the
// 4-wave 128-query variant, two workgroups per compute unit; about 512
// workgroups in all was the fastest count on every few-head shape measured
// on MI355X (8 to 16 ranges at 32 to 128 query tiles over 16384 to 32768
// keys, 9-14 % faster than about 256 with the 8-wave variant).
constexpr int kFusedSplitBelow = 256;         // split when fewer workgroups than this
constexpr int kFusedSplitTargetGroups = 512;  // up to about this many workgroups
constexpr int kFusedSplitMinKeys = 1024;      // keys per range, at least
constexpr int kFusedSplitMinTotal = 4096;     // keys per row, at least, to split at all
constexpr int kFusedSplitMax = 64;            // ranges, at most

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [B,H,S,d], [B,S,H,d], or groups of g heads (1 <= g, g divides H)
bool layout_ok(int layout, int H) {
    if (layout == ATTN_LAYOUT_BHSD || layout == ATTN_LAYOUT_BSHD) return true;
    if ((layout & ~0xffff) != ATTN_LAYOUT_SPLIT(0)) return false;
    const int g = layout & 0xffff;
    return g >= 1 && H % g == 0;
}

int check_shape(int B, int H, int Sq, int Sk, int d, int layout, int dtype) {
    if (B < 1 || H < 1 || Sq < 1 || Sk < 1) return ATTN_E_SHAPE;
    if (d != 64 && d != 128) return ATTN_E_UNSUPPORTED;
    if (!layout_ok(layout, H)) return ATTN_E_UNSUPPORTED;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
    // every row index (b*H + h)*S + s and every workgroup count fits in int32
    const int64_t rows_q = (int64_t)B * H * Sq;
    const int64_t rows_k = (int64_t)B * H * Sk;
    if (rows_q > INT_MAX || rows_k > INT_MAX) return ATTN_E_SHAPE;
    return ATTN_OK;
}

}  // namespace

namespace attn {
int check_fwd_call(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   int B, int H, int Sq, int Sk, int d, float scale, int layout, int dtype,
                   const int32_t* kv_len) {
    if (!q || !k || !v || !o) return ATTN_E_NULLPTR;
    int rc = check_shape(B, H, Sq, Sk, d, layout, dtype);
    if (rc != ATTN_OK) return rc;
    if (!std::isfinite(scale) || scale < 0.f) return ATTN_E_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return ATTN_E_ALIGN;
    if (!aligned(lse, 4) || !aligned(kv_len, 4)) return ATTN_E_ALIGN;
    return ATTN_OK;
}
}  // namespace attn

namespace {

using attn::check_fwd_call;

// Key splits for the fused kernel (16-bit types, Sq > kSplitMaxQueries);
// Sk is the keys a row can see
int plan_fused_splits(int B, int H, int Sq, int Sk, int dtype) {
    if (dtype == ATTN_F32 || Sk < kFusedSplitMinTotal) return 1;
    const int64_t groups = (int64_t)B * H * ((Sq + 127) / 128);
    if (groups >= kFusedSplitBelow) return 1;
    int64_t n = (kFusedSplitTargetGroups + groups - 1) / groups;
    if (n > Sk / kFusedSplitMinKeys) n = Sk / kFusedSplitMinKeys;
    if (n > kFusedSplitMax) n = kFusedSplitMax;
    return n >= 2 ? (int)n : 1;
}

int plan_splits(int B, int H, int Sq, int Sk, int dtype, int causal) {
    // a causal row i sees keys 0 .. i: no row sees more than Sq keys
    if (causal && Sq < Sk) Sk = Sq;
    if (Sq > kSplitMaxQueries) return plan_fused_splits(B, H, Sq, Sk, dtype);
    const int64_t rows = (int64_t)B * H * Sq;
    int64_t n = (kSplitTargetGroups + rows - 1) / rows;
    if (n < Sk / kSplitMaxKeys) n = Sk / kSplitMaxKeys;
    if (n > Sk / kSplitMinKeys) n = Sk / kSplitMinKeys;
    if (n > 256) n = 256;
    // even at one split per row the split kernels beat the fused kernel
    // here; only very short key ranges stay fused (one launch)
    if (n < 2) return Sk >= 2 * kSplitMinKeys ? 2 : 1;
    return (int)n;
}

attn::FwdArgs make_args(const void* q, const void* k, const void* v, void* o, float* lse,
                        int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                        int dtype, const int32_t* kv_len) {
    attn::FwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.kv_len = kv_len;
    a.B = B;
    a.H = H;
    a.Sq = Sq;
    a.Sk = Sk;
    a.d = d;
    a.scale = scale;
    a.causal = causal != 0;
    a.layout = layout;
    a.dtype = dtype;
    return a;
}

int status_of(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_E_HIP; }

}  // namespace

extern "C" {

int attn_fwd_plan(int B, int H, int Sq, int Sk, int d, int dtype, int causal, int* n_split) {
    if (!n_split) return ATTN_E_NULLPTR;
    int rc = check_shape(B, H, Sq, Sk, d, ATTN_LAYOUT_BHSD, dtype);
    if (rc != ATTN_OK) return rc;
    *n_split = plan_splits(B, H, Sq, Sk, dtype, causal);
    return ATTN_OK;
}

size_t attn_splitk_workspace_size(int B, int H, int Sq, int d, int n_split) {
    if (n_split < 1 || check_shape(B, H, Sq, 1, d, ATTN_LAYOUT_BHSD, ATTN_F32) != ATTN_OK) return 0;
    return attn::splitk_workspace_bytes(B, H, Sq, d, n_split);
}

size_t attn_fwd_workspace_size(int B, int H, int Sq, int Sk, int d, int dtype, int causal) {
    if (check_shape(B, H, Sq, Sk, d, ATTN_LAYOUT_BHSD, dtype) != ATTN_OK) return 0;
    const int n = plan_splits(B, H, Sq, Sk, dtype, causal);
    return n > 1 ? attn::splitk_workspace_bytes(B, H, Sq, d, n) : 0;
}

int attn_fwd_splitk(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                    int dtype, const int32_t* kv_len, int n_split, void* workspace,
                    size_t workspace_bytes, void* stream) {
    int rc = check_fwd_call(q, k, v, o, lse, B, H, Sq, Sk, d, scale, layout, dtype, kv_len);
    if (rc != ATTN_OK) return rc;
    if (n_split < 1 || (int64_t)B * H * Sq * n_split > INT_MAX) return ATTN_E_SHAPE;
    const size_t need = attn::splitk_workspace_bytes(B, H, Sq, d, n_split);
    if (!workspace || workspace_bytes < need) return ATTN_E_WORKSPACE;
    if (!aligned(workspace, 16)) return ATTN_E_ALIGN;
    const attn::FwdArgs a = make_args(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, layout, dtype, kv_len);
    return status_of(attn::run_splitk(a, n_split, workspace, static_cast<hipStream_t>(stream)));
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
             int dtype, const int32_t* kv_len, void* workspace, size_t workspace_bytes,
             void* stream) {
    int rc = check_fwd_call(q, k, v, o, lse, B, H, Sq, Sk, d, scale, layout, dtype, kv_len);
    if (rc != ATTN_OK) return rc;
    const int n = plan_splits(B, H, Sq, Sk, dtype, causal);
    if (n > 1 && Sq <= kSplitMaxQueries)
        return attn_fwd_splitk(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, layout, dtype, kv_len, n,
                               workspace, workspace_bytes, stream);
    return attn_fwd_tiled(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, layout, dtype, kv_len, -1, n,
                          workspace, workspace_bytes, stream);
}

int attn_fwd_tile_count(int d, int dtype) {
    if (check_shape(1, 1, 1, 1, d, ATTN_LAYOUT_BHSD, dtype) != ATTN_OK) return 0;
    return attn::prefill_tile_count(d, dtype);
}

int attn_fwd_tile_info(int d, int dtype, int tile, attn_tile_info* info) {
    if (!info) return ATTN_E_NULLPTR;
    int rc = check_shape(1, 1, 1, 1, d, ATTN_LAYOUT_BHSD, dtype);
    if (rc != ATTN_OK) return rc;
    attn::TileInfo t;
    if (!attn::prefill_tile_info(d, dtype, tile, &t)) return ATTN_E_ARG;
    info->rows = t.rows;
    info->keys = t.keys;
    info->waves = t.waves;
    info->stages = t.stages;
    info->lds_bytes = t.lds_bytes;
    return ATTN_OK;
}

int attn_fwd_tile_choice(int B, int H, int Sq, int Sk, int d, int dtype, int causal, int* tile) {
    if (!tile) return ATTN_E_NULLPTR;
    int rc = check_shape(B, H, Sq, Sk, d, ATTN_LAYOUT_BHSD, dtype);
    if (rc != ATTN_OK) return rc;
    const int n = plan_splits(B, H, Sq, Sk, dtype, causal);
    *tile = attn::prefill_tile_choice(B, H, Sq, Sk, d, dtype, causal != 0,
                                      Sq > kSplitMaxQueries ? n : 1);
    return ATTN_OK;
}

int attn_fwd_tiled(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                   int dtype, const int32_t* kv_len, int tile, int n_split, void* workspace,
                   size_t workspace_bytes, void* stream) {
    int rc = check_fwd_call(q, k, v, o, lse, B, H, Sq, Sk, d, scale, layout, dtype, kv_len);
    if (rc != ATTN_OK) return rc;
    if (tile < -1 || tile >= attn::prefill_tile_count(d, dtype) || n_split < 1) return ATTN_E_ARG;
    if (n_split > 1) {
        if (dtype == ATTN_F32) return ATTN_E_UNSUPPORTED;
        // record indices and key-range ends (ranges are whole 64-key tiles) fit in int32
        if ((int64_t)B * H * Sq * n_split > INT_MAX || (int64_t)Sk + (int64_t)n_split * 64 > INT_MAX)
            return ATTN_E_SHAPE;
        const size_t need = attn::splitk_workspace_bytes(B, H, Sq, d, n_split);
        if (!workspace || workspace_bytes < need) return ATTN_E_WORKSPACE;
        if (!aligned(workspace, 16)) return ATTN_E_ALIGN;
    }
    attn::FwdArgs a = make_args(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, layout, dtype, kv_len);
    a.tile = tile;
    a.n_split = n_split;
    a.ws = n_split > 1 ? workspace : nullptr;
    return status_of(attn::run_prefill(a, static_cast<hipStream_t>(stream)));
}

size_t attn_naive_scratch_size(int B, int H, int Sq, int Sk, int dtype) {
    if (check_shape(B, H, Sq, Sk, 64, ATTN_LAYOUT_BHSD, dtype) != ATTN_OK) return 0;
    return attn::naive_scratch_bytes(B, H, Sq, Sk, dtype);
}

int attn_fwd_naive(const void* q, const void* k, const void* v, void* o, float* lse,
                   int B, int H, int Sq, int Sk, int d, float scale, int causal, int layout,
                   int dtype, const int32_t* kv_len, void* scratch, size_t scratch_bytes,
                   void* stream) {
    int rc = check_fwd_call(q, k, v, o, lse, B, H, Sq, Sk, d, scale, layout, dtype, kv_len);
    if (rc != ATTN_OK) return rc;
    const size_t need = attn::naive_scratch_bytes(B, H, Sq, Sk, dtype);
    if (!scratch || scratch_bytes < need) return ATTN_E_WORKSPACE;
    if (!aligned(scratch, 16)) return ATTN_E_ALIGN;
    const attn::FwdArgs a = make_args(q, k, v, o, lse, B, H, Sq, Sk, d, scale, causal, layout, dtype, kv_len);
    return status_of(attn::run_naive(a, scratch, static_cast<hipStream_t>(stream)));
}

int attn_qkv_proj(const void* x, const void* w, void* q, void* k, void* v, int B, int S, int D,
                  int H, int d, int layout, int dtype, void* stream) {
    if (!x || !w || !q || !k || !v) return ATTN_E_NULLPTR;
    if (H < 1) return ATTN_E_SHAPE;
    if (!layout_ok(layout, H)) return ATTN_E_UNSUPPORTED;
    if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
    if (B < 1 || S < 1 || H < 1 || D < 64 || D % 64 != 0 || d < 8 || d % 8 != 0) return ATTN_E_SHAPE;
    if ((int64_t)B * S > INT_MAX || (int64_t)3 * H * d > INT_MAX) return ATTN_E_SHAPE;
    if (!aligned(x, 16) || !aligned(w, 16) || !aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16))
        return ATTN_E_ALIGN;
    attn::QkvArgs a;
    a.x = x;
    a.w = w;
    a.q = q;
    a.k = k;
    a.v = v;
    a.B = B;
    a.S = S;
    a.D = D;
    a.H = H;
    a.d = d;
    a.layout = layout;
    a.dtype = dtype;
    return status_of(attn::run_qkv_proj(a, static_cast<hipStream_t>(stream)));
}

int attn_qkv_proj_tiling(int B, int S, int H, int d, int n_cu, int* tiling) {
    if (!tiling) return ATTN_E_NULLPTR;
    if (B < 1 || S < 1 || H < 1 || d < 1 || n_cu < 1) return ATTN_E_SHAPE;
    if ((int64_t)B * S > INT_MAX || (int64_t)3 * H * d > INT_MAX) return ATTN_E_SHAPE;
    *tiling = attn::qkv_proj_tiling(B * S, 3 * H * d, n_cu);
    return ATTN_OK;
}

int attn_softmax_rows(const void* x, void* y, float* lse, int64_t rows, int n, float scale,
                      int dtype, int mode, void* stream) {
    if (!x || !y) return ATTN_E_NULLPTR;
    if (dtype != ATTN_F32 && dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_E_UNSUPPORTED;
    if (mode != ATTN_SOFTMAX_ONLINE && mode != ATTN_SOFTMAX_THREE_PASS) return ATTN_E_UNSUPPORTED;
    const int per16 = dtype == ATTN_F32 ? 4 : 8;  // elements per 16 bytes
    if (rows < 1 || rows > INT_MAX || n < 1 || n % per16 != 0) return ATTN_E_SHAPE;
    if (!std::isfinite(scale) || scale < 0.f) return ATTN_E_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(lse, 4)) return ATTN_E_ALIGN;
    attn::SoftmaxArgs a;
    a.x = x;
    a.y = y;
    a.lse = lse;
    a.rows = rows;
    a.n = n;
    a.scale = scale;
    a.dtype = dtype;
    a.mode = mode;
    return status_of(attn::run_softmax_rows(a, static_cast<hipStream_t>(stream)));
}

const char* attn_status_string(int status) {
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULLPTR: return "a required pointer is NULL";
    case ATTN_E_SHAPE: return "invalid shape: sizes must be >= 1 (projection: D a multiple of 64, d of 8) and fit";
    case ATTN_E_UNSUPPORTED: return "unsupported head size (64 or 128), layout or dtype";
    case ATTN_E_ALIGN: return "misaligned pointer (tensors and workspaces 16 bytes, lse and kv_len 4 bytes)";
    case ATTN_E_WORKSPACE: return "workspace or scratch missing or too small";
    case ATTN_E_HIP: return "the HIP runtime reported an error at launch";
    case ATTN_E_ARG: return "invalid argument: scale negative, NaN or infinite, tile variant out of range, or n_split < 1";
    case ATTN_E_SCRATCH_LIMIT: return "the call needs more workspace than attn_fwd_noalloc's static buffer holds (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
    }
}

int attn_version(void) { return kVersion; }

}  // extern "C"

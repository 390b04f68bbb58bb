// Host-side launchers of the libattn kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Arguments of one forward call after validation (see include/attn.h).
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* kv_len;
    int B, H, Sq, Sk, d;
    float scale;
    int causal;
    int layout;     // 0 = [B,H,S,d], 1 = [B,S,H,d], 0x10000 | g = groups of g heads
    int dtype;      // 0 = fp32, 1 = fp16, 2 = bf16
    int tile = -1;  // fused kernel's tile variant; -1 = the tuned table's choice
    // fused kernel over key splits: n_split > 1 writes per-split (m, l, o)
    // records to `ws` (the split-K layout) and merges them
    int n_split = 1;
    void* ws = nullptr;
};

// The host-side checks of attn_fwd's arguments (status codes of attn.h).
int check_fwd_call(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   int B, int H, int Sq, int Sk, int d, float scale, int layout, int dtype,
                   const int32_t* kv_len);

// Fused single-kernel forward (any shape); 16-bit inputs go to run_prefill16.
hipError_t run_prefill(const FwdArgs& a, hipStream_t stream);
hipError_t run_prefill16(const FwdArgs& a, hipStream_t stream);

// Tile variants of the fused kernel (as attn_tile_info in attn.h).
struct TileInfo {
    int rows, keys, waves, stages, lds_bytes;
};
int prefill_tile_count(int d, int dtype);
bool prefill_tile_info(int d, int dtype, int tile, TileInfo* out);
// the variant the fused kernel runs for this shape over n_split key ranges
int prefill_tile_choice(int B, int H, int Sq, int Sk, int d, int dtype, int causal, int n_split);
int prefill16_tile_count(int d);
bool prefill16_tile_info(int d, int tile, TileInfo* out);
int prefill16_tile_choice(int B, int H, int Sq, int Sk, int d, int causal, int n_split);

// Split-over-keys forward: partial kernel + merge kernel.
size_t splitk_workspace_bytes(int B, int H, int Sq, int d, int n_split);
hipError_t run_splitk(const FwdArgs& a, int n_split, void* workspace, hipStream_t stream);
// The merge kernel alone, over records another kernel wrote.
hipError_t run_splitk_merge(const FwdArgs& a, int n_split, const void* workspace, hipStream_t stream);

// QKV projection: x [B,S,D] times the out-major weight [3*H*d, D] into q, k, v.
struct QkvArgs {
    const void* x;
    const void* w;
    void* q;
    void* k;
    void* v;
    int B, S, D, H, d;
    int layout;  // as FwdArgs::layout
    int dtype;   // 1 = fp16, 2 = bf16
};
hipError_t run_qkv_proj(const QkvArgs& a, hipStream_t stream);
// Tiling of the QKV projection for M tokens and N columns on n_cu CUs (0 or 1).
int qkv_proj_tiling(int M, int N, int n_cu);

// Row softmax of x [rows, n] (mode 0 online, 1 three-pass).
struct SoftmaxArgs {
    const void* x;
    void* y;
    float* lse;
    int64_t rows;
    int n;
    float scale;
    int dtype;
    int mode;
};
hipError_t run_softmax_rows(const SoftmaxArgs& a, hipStream_t stream);

// Unfused three-kernel baseline.
size_t naive_scratch_bytes(int B, int H, int Sq, int Sk, int dtype);
hipError_t run_naive(const FwdArgs& a, void* scratch, hipStream_t stream);

}  // namespace attn

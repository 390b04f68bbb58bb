// Device helpers shared by the libattn kernels (gfx950, wave64).
//
// Matrix-core conventions used throughout (CDNA 32x32 MFMA family):
//   A operand: lane l supplies row  (l % 32) of the 32 x K block,
//   B operand: lane l supplies column (l % 32) of the K x 32 block,
//   in both cases the contraction slots held by lane half (l / 32). The
//   32 x 32 fp32 result sits in 16 registers per lane: register r of lane l
//   is element [8*(r/4) + 4*(l/32) + r%4][l % 32].
// Only that result layout and the row/column ownership matter: A and B read
// their contraction slots through the same (lane half, element) numbering,
// so the order of the slots inside the instruction never changes the sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace attn {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Storage tags: the element type of q, k, v, o.
struct BF16 { typedef uint16_t storage; static constexpr int bytes = 2; };
struct F16  { typedef uint16_t storage; static constexpr int bytes = 2; };
struct F32  { typedef float storage;    static constexpr int bytes = 4; };

// ---- conversions -----------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
// Two floats to a packed pair of 16-bit values, round to nearest even.
template <typename Tag> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}
// Low / high 16-bit element of a packed pair, as float.
template <typename Tag> __device__ __forceinline__ float lo16(uint32_t w);
template <typename Tag> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float lo16<BF16>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float hi16<BF16>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <> __device__ __forceinline__ float lo16<F16>(uint32_t w) { return f16_to_f32(w & 0xffffu); }
template <> __device__ __forceinline__ float hi16<F16>(uint32_t w) { return f16_to_f32(w >> 16); }

// ---- matrix-core products: 32x32 fp32 block += A(32 x K) * B(K x 32) -------
// 16-bit inputs: K = 16, 8 elements (one u32x4) per lane and operand.
template <typename Tag> __device__ __forceinline__ f32x16 mfma16(u32x4 a, u32x4 b, f32x16 c);
template <> __device__ __forceinline__ f32x16 mfma16<BF16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x16 mfma16<F16>(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// 16x16 fp32 block += A(16 x 32) * B(32 x 16), 16-bit inputs, 8 elements per
// lane and operand: lane l supplies A row (l % 16), contraction slots
// 8*(l/16) .. +7, and B column (l % 16), the same slots; result register j
// of lane l is element [4*(l/16) + j][l % 16].
template <typename Tag> __device__ __forceinline__ f32x4 mfma16x16(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma16x16<BF16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma16x16<F16>(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
// fp32 inputs: K = 2, one element per lane and operand.
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Base-2 exponential on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of the lane in the other half of the wave (lane ^ 32).
__device__ __forceinline__ float swap_halves(float x) {
    const uint32_t u = __float_as_uint(x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // lanes 0-31 receive lanes 32-63 in r[1]; lanes 32-63 receive lanes 0-31 in r[0]
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Row (key) index held by result register r in lane half h: 8*(r/4) + 4*h + r%4.
__device__ __forceinline__ constexpr int blk_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// ---- addressing -------------------------------------------------------------
// Element offsets in one tensor of B x H heads x S rows x d, for the three
// layouts: heads in groups of g, [B, H/g, S, g, d]. g = 1 is [B,H,S,d]
// (heads outermost), g = H is [B,S,H,d] (heads interleaved per token), and
// anything between is the "Split" head-group layout.
struct Strides {
    int64_t b;    // between batches
    int64_t grp;  // between head groups
    int64_t s;    // between consecutive rows (tokens) of one head
    int hd;       // between heads of one group
    int g;        // heads per group
    __host__ __device__ int64_t head(int bi, int h) const {
        return bi * b + (int64_t)(h / g) * grp + (int64_t)(h % g) * hd;
    }
};

// Layout codes (see include/attn.h): 0 = [B,H,S,d], 1 = [B,S,H,d],
// 0x10000 | g = groups of g heads. Returns the heads per group.
__host__ __device__ inline int layout_group(int layout, int H) {
    if (layout == 0) return 1;
    if (layout == 1) return H;
    return layout & 0xffff;
}

__host__ __device__ inline Strides make_strides(int layout, int H, int S, int d) {
    const int g = layout_group(layout, H);
    Strides st;
    st.b = (int64_t)S * H * d;
    st.grp = (int64_t)S * g * d;
    st.s = (int64_t)g * d;
    st.hd = d;
    st.g = g;
    return st;
}

// Transposed LDS store of two consecutive 16-bit key rows (keys 2*pr and
// 2*pr+1), 8 elements each starting at d = 8*cc: element d of both rows goes
// to row d of Vt as one 32-bit word at column 2*pr. vrow = Vt row length.
__device__ __forceinline__ void store_pair_transposed(uint16_t* Vt, int vrow, int cc, int pr,
                                                      const u32x4& r0, const u32x4& r1) {
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
        const uint32_t a0 = r0[wd], a1 = r1[wd];
        const uint32_t lo = (a0 & 0xffffu) | (a1 << 16);      // d = 8cc + 2wd
        const uint32_t hi = (a0 >> 16) | (a1 & 0xffff0000u);  // d = 8cc + 2wd + 1
        *reinterpret_cast<uint32_t*>(Vt + (cc * 8 + 2 * wd) * vrow + 2 * pr) = lo;
        *reinterpret_cast<uint32_t*>(Vt + (cc * 8 + 2 * wd + 1) * vrow + 2 * pr) = hi;
    }
}

template <typename Tag> __device__ __forceinline__ typename Tag::storage to_storage(float x);
template <> __device__ __forceinline__ uint16_t to_storage<BF16>(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
template <> __device__ __forceinline__ uint16_t to_storage<F16>(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}
template <> __device__ __forceinline__ float to_storage<F32>(float x) { return x; }

__device__ __forceinline__ int clamp_len(const int32_t* kv_len, int b, int Sk) {
    if (kv_len == nullptr) return Sk;
    int n = kv_len[b];
    return n < 0 ? 0 : (n > Sk ? Sk : n);
}

}  // namespace attn

// Internal helpers shared by the gfx950 kernels of the paged-KV library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

#include "nv_paged.h"

namespace nvp {

constexpr int kWave = 64;
constexpr int kHeadDim = 128;  // the only head size this library implements

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// log2(e): exp(x) = exp2(x * log2(e)); the kernels fold it into the softmax scale.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// A packed bf16 pair as the operand type of the bf16 dot builtins. Takes the word by value:
// applying __builtin_bit_cast directly to a vector-element expression (x[e]) is miscompiled by
// this compiler (every element reads as element 0), a scalar copy is not.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t word) {
    return __builtin_bit_cast(bf16x2, word);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over each row of 16 lanes via DPP rotations; every lane of the row gets the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));
    return x;
}

// Pool row of logical key j of a sequence: its block id times the block size plus the offset.
__device__ __forceinline__ int64_t key_row(const int32_t *table, int32_t j, int32_t bs,
                                           int32_t bs_shift) {
    int32_t lb, off;
    if (bs_shift >= 0) {
        lb = j >> bs_shift;
        off = j & (bs - 1);
    } else {
        lb = j / bs;
        off = j - lb * bs;
    }
    return (int64_t)table[lb] * bs + off;
}

__device__ __forceinline__ float wave_max(float x) {
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Launch through hipLaunchKernel so the launch's own status is returned (no reliance on, or
// clearing of, the thread's sticky last-error state).
template <typename... KArgs, typename... Args>
inline nv_status launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds_bytes,
                        hipStream_t stream, Args &&...args) {
    std::tuple<KArgs...> values(std::forward<Args>(args)...);
    void *ptrs[sizeof...(KArgs)];
    std::apply([&](auto &...v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void *>(&v)), ...);
    }, values);
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, ptrs,
                                   lds_bytes, stream);
    return e == hipSuccess ? NV_OK : NV_ERR_LAUNCH;
}

}  // namespace nvp

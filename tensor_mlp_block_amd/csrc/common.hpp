// common.hpp -- device helpers shared by the gfx950 kernels of libmlptp.so.
//
// Pages cited, as [tag section]:
//   [Z] zwjcode.cn, "一层 MLP 太宽而放不下时怎样切？列并行、行并行与块尾归约"
//   [C] charliedreemur.github.io, "TP:Column / Row Parallel Linear 怎么切? MLP 和 attention 怎么切?"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mlptp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

enum ActCode : int {
    kActIdentity = 0,
    kActRelu = 1,
    kActGeluTanh = 2,
    kActGeluErf = 3,
    kActGeluSigmoid = 4,
};

// bf16 is carried as its 16-bit pattern; widening is exact.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f)
{
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

// Two values rounded and packed by one v_cvt_pk_bf16_f32 (lo in bits 0-15). Written as
// two scalar conversions joined by a shift and an or, the compiler emits four instructions.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Logistic function 1 / (1 + e^-x), stable at both ends (e^-x -> inf gives 0, -> 0 gives 1).
// The reciprocal is the hardware one (v_rcp_f32, about 1 ulp) rather than a correctly rounded
// division, which costs about ten instructions; every result of it is rounded to bf16 or feeds
// a tolerance of 1e-2.
__device__ __forceinline__ float sigmoidf_(float x)
{
    return __builtin_amdgcn_rcpf(1.0f + __expf(-x));
}

// SiLU(z) = z * sigmoid(z), the gate nonlinearity of the gated MLP.
__device__ __forceinline__ float silu_f(float z) { return z * sigmoidf_(z); }

// GELU, tanh form: 0.5 z (1 + tanh(u)) with u = sqrt(2/pi) (z + 0.044715 z^3). Since
// 0.5 (1 + tanh(u)) equals the logistic function at 2u, it is evaluated as z * sigmoid(2u)
// = z / (1 + 2^t), t = -2 log2(e) u, which needs one exponential and saturates cleanly for
// large |z|. The constants are kept in double and folded before rounding to float.
constexpr double kSqrt2OverPiD = 0.7978845608028654;
constexpr double kTanhCubicD = 0.044715;
constexpr double kLog2eD = 1.4426950408889634;
// -2 log2(e) sqrt(2/pi) and that times 0.044715: the GELU-tanh exponent in base 2.
constexpr float kGeluExp2C1 = (float)(-2.0 * kLog2eD * kSqrt2OverPiD);
constexpr float kGeluExp2C3 = (float)(-2.0 * kLog2eD * kSqrt2OverPiD * kTanhCubicD);
// 2 sqrt(2/pi) and 2 sqrt(2/pi) 3 (0.044715): twice the derivative of the tanh argument.
constexpr float kGeluDu2C1 = (float)(2.0 * kSqrt2OverPiD);
constexpr float kGeluDu2C3 = (float)(2.0 * kSqrt2OverPiD * 3.0 * kTanhCubicD);
constexpr float kSigmoidScale = 1.702f;
constexpr float kInvSqrt2 = 0.7071067811865476f;
constexpr float kInvSqrt2Pi = 0.3989422804014327f;

// phi(z) [Z 02]: elementwise, so each shard applies it to its own columns with no exchange.
// The activation is a compile-time parameter so a kernel inlines only its own form.
template <int ACT>
__device__ __forceinline__ float act_fwd(float z)
{
    if constexpr (ACT == kActRelu) {
        return z > 0.0f ? z : 0.0f;
    } else if constexpr (ACT == kActGeluTanh) {
        // z sigmoid(2u) = z / (1 + 2^t), t = -2 log2(e) u = z (c1 + c3 z^2): the constants are
        // folded so the exponent is one multiply-add and one multiply, and the power of two is
        // the hardware's (v_exp_f32). z -> -inf gives 2^t = inf and -0; z -> +inf gives z.
        const float t = z * fmaf(z * z, kGeluExp2C3, kGeluExp2C1);
        return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
    } else if constexpr (ACT == kActGeluErf) {
        // z Phi(z), Phi(z) = erfc(-z / sqrt 2) / 2. Written as 1 + erf(z / sqrt 2), the sum
        // cancels for negative z and keeps none of the digits of results below fp32's epsilon
        // (z = -8: an absolute error of 2e-7 on a value of -5e-15).
        return 0.5f * z * erfcf(-z * kInvSqrt2);
    } else if constexpr (ACT == kActGeluSigmoid) {
        return z * sigmoidf_(kSigmoidScale * z);
    } else {
        return z;
    }
}

// phi'(z), used by the backward "through the local activation" [Z 06]. ReLU'(0) = 0.
template <int ACT>
__device__ __forceinline__ float act_grad(float z)
{
    if constexpr (ACT == kActRelu) {
        return z > 0.0f ? 1.0f : 0.0f;
    } else if constexpr (ACT == kActGeluTanh) {
        // s = sigmoid(2u) = 0.5 (1 + tanh u) = 1 / (1 + 2^t) with t as in act_fwd, and
        // 0.5 (1 - tanh^2 u) = 2 s (1 - s): phi' = s + z s (1 - s) (2 du), where
        // 2 du = 2 sqrt(2/pi) (1 + 3 (0.044715) z^2) is one multiply-add of z^2.
        const float z2 = z * z;
        const float t = z * fmaf(z2, kGeluExp2C3, kGeluExp2C1);
        const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(t));
        const float du2 = fmaf(z2, kGeluDu2C3, kGeluDu2C1);
        return fmaf(z * s * (1.0f - s), du2, s);
    } else if constexpr (ACT == kActGeluErf) {
        const float cdf = 0.5f * erfcf(-z * kInvSqrt2);
        return cdf + z * kInvSqrt2Pi * __expf(-0.5f * z * z);
    } else if constexpr (ACT == kActGeluSigmoid) {
        const float s = sigmoidf_(kSigmoidScale * z);
        return s + kSigmoidScale * z * s * (1.0f - s);
    } else {
        return 1.0f;
    }
}

// Calls f(std::integral_constant<int, ACT>) for the runtime activation code `act`.
template <class F>
inline void with_act(int act, F&& f)
{
    switch (act) {
    case kActRelu: f(std::integral_constant<int, kActRelu>{}); break;
    case kActGeluTanh: f(std::integral_constant<int, kActGeluTanh>{}); break;
    case kActGeluErf: f(std::integral_constant<int, kActGeluErf>{}); break;
    case kActGeluSigmoid: f(std::integral_constant<int, kActGeluSigmoid>{}); break;
    default: f(std::integral_constant<int, kActIdentity>{}); break;
    }
}

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace mlptp

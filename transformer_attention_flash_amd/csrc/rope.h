// rope.h -- GPT-NeoX half-split partial rotary position embedding, applied by
// the kernels to rows as they load them.
//
// Semantics: trustformers-core 0.2.0 src/gpu_ops/cuda/oxicuda/attention.rs,
// `rope_neox_gpu_to_gpu` and its CPU helper `rope_reference`; realizar 0.8.5
// src/cuda/executor/cache_from_cache_from_kv_cache.rs, `apply_rope_to_buffer`
// (the rotary_ndims = head_dim case, with base = rope theta).  Within each
// head, dim i < half = rotary_ndims / 2 is paired with dim i + half and the
// pair is turned by the angle pos * base^(-2i / rotary_ndims):
//   y_i        = x_i cos a - x_{i+half} sin a
//   y_{i+half} = x_i sin a + x_{i+half} cos a
// and dims at or past rotary_ndims are left as they are.
//
// Precision: the angle of pair i is kept in turns (revolutions).  The host
// computes turns_i = base^(-2i/rotary_ndims) / (2 pi) in double once per call;
// a kernel forms pos * turns_i in double, drops the whole turns, and only the
// remaining fraction (|f| <= 1/2) goes to single precision for sin(2 pi f) and
// cos(2 pi f).  The angle error is then about 1e-7 rad at any int32 position,
// where an angle formed in single precision would be off by up to
// ulp(pos) ~ 2e-3 rad near position 32768.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"

namespace attn {

constexpr int kMaxRopeHalf = 64;  // head_dim <= 128

struct RopeParams {
    int32_t rot;   // rotary_ndims: 0 (off) or a multiple of 8 up to head_dim
    int32_t half;  // rot / 2
    double turns[kMaxRopeHalf];  // revolutions per position of pair i
};

// Host: the per-pair turn rates for rotary_ndims `rot` and base `theta`
// (validated by the caller: rot % 8 == 0, 0 <= rot <= 128, theta > 0 finite).
inline RopeParams make_rope(int32_t rot, float theta) {
    RopeParams r{};
    r.rot = rot;
    r.half = rot / 2;
    const double two_pi = 6.283185307179586476925286766559;
    for (int32_t i = 0; i < r.half; ++i)
        r.turns[i] = pow((double)theta, -2.0 * (double)i / (double)rot) / two_pi;
    return r;
}

// sin and cos of the angle of a pair turning at `turns` revolutions per
// position, at position pos.
__device__ __forceinline__ void rope_sincos(int32_t pos, double turns, float &s, float &c) {
    const double t = (double)pos * turns;
    const double f = t - rint(t);
    sincospif((float)(2.0 * f), &s, &c);
}

// Rotates four dims given their partners and the sin/cos of their angles:
// `low` dims (i < half) take x cos - partner sin, the others partner sin + x cos.
__device__ __forceinline__ f32x4 rope_apply4(f32x4 x, f32x4 partner, bool low, const float *sn,
                                             const float *cs) {
    f32x4 y;
#pragma unroll
    for (int c = 0; c < 4; ++c) y[c] = low ? x[c] * cs[c] - partner[c] * sn[c] : partner[c] * sn[c] + x[c] * cs[c];
    return y;
}

// The four dims l0 .. l0+3 (l0 % 4 == 0) of one head row at position pos,
// rotated.  x holds those dims; partner holds dims l0 + half .. (l0 < half)
// or l0 - half .. (half <= l0 < rot); partner is ignored for l0 >= rot.
__device__ __forceinline__ f32x4 rope_rotate4(f32x4 x, f32x4 partner, int l0, int32_t pos,
                                              const RopeParams &rp) {
    if (l0 >= rp.rot) return x;
    const bool low = l0 < rp.half;
    const int i0 = low ? l0 : l0 - rp.half;
    float sn[4], cs[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) rope_sincos(pos, rp.turns[i0 + c], sn[c], cs[c]);
    return rope_apply4(x, partner, low, sn, cs);
}

}  // namespace attn

// Device helpers shared by the gfx950 kernels of libssm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt immediate for vmcnt(0) with expcnt and lgkmcnt left at their maximum (no wait).
constexpr int kWaitVmcnt0 = 0x0F70;

// bfloat16 storage: the 16 high bits of an IEEE float.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (finite inputs; NaN stays NaN-like).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// Hardware reciprocal (v_rcp_f32, about 1 ulp).
__device__ __forceinline__ float rcp_fast(float v) { return __builtin_amdgcn_rcpf(v); }

// z * sigmoid(z) with the hardware exp and reciprocal; exp2 overflows to +inf for very
// negative z, which gives -0 (the limit).
__device__ __forceinline__ float silu(float zv) {
  return zv * rcp_fast(1.0f + exp2_fast(-zv * kLog2e));
}

// sigmoid(v) = 1 / (1 + e^-v) with the hardware exp and reciprocal (0 and 1 in the limits).
__device__ __forceinline__ float sigmoid_fast(float v) {
  return rcp_fast(1.0f + exp2_fast(-v * kLog2e));
}

// Raw buffer access. A buffer descriptor holds a base address and a size in bytes; a load at an
// offset at or past the size returns zero and a store there is dropped. The tile loops build one
// descriptor per tile and tensor (scalar work) whose size ends with the tile's last row inside
// the segment, so the rows of a ragged last tile read as zeros and their stores vanish with no
// per-lane row tests, and the lanes pass only a 32-bit byte offset. Word 3 selects the 32-bit
// data format with untyped (raw) addressing.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRawRsrcWord3 = 0x00020000;

// base and bytes are uniform over the wave; readfirstlane says so to the compiler (otherwise a
// value it cannot prove uniform makes it wrap each buffer access in a loop over distinct values).
__device__ __forceinline__ Rsrc make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, __builtin_amdgcn_readfirstlane(bytes), kRawRsrcWord3);
}
__device__ __forceinline__ void buf_load(Rsrc r, uint32_t off, uint2& out) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  out = make_uint2(v[0], v[1]);
}
__device__ __forceinline__ void buf_load(Rsrc r, uint32_t off, uint4& out) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  out = make_uint4(v[0], v[1], v[2], v[3]);
}

// softplus(u) = log(1 + e^u) = max(u, 0) + log1p(e) with e = exp(-|u|) in (0, 1].
//  * e: the base-2 exponent t = -|u| log2(e) is carried as t_hi + t_lo (t_lo from an fma and the
//    tail of log2(e)), and exp2(t_hi + t_lo) = exp2(t_hi) (1 + t_lo ln 2), so the rounding of
//    the argument does not grow with |u|.
//  * log1p(e) = 2 atanh(s) with s = e / (2 + e) in (0, 1/3], summed as the odd power series
//    2 s (1 + s^2/3 + s^4/5 + ... + s^12/13); the omitted tail is below 2^-24 relative for
//    s <= 1/3. About a dozen VALU operations and two hardware transcendentals.
// Inputs below -150 give 0 (the true value underflows), +inf gives +inf, NaN stays NaN.
__device__ __forceinline__ float softplus_f32(float u) {
  constexpr float kLog2eTail = 1.925963033e-8f;  // log2(e) - (float)log2(e)
  constexpr float kLn2 = 0.6931471806f;
  const float x = fmaxf(-fabsf(u), -150.0f);
  const float t_hi = x * kLog2e;
  const float t_lo = fmaf(x, kLog2e, -t_hi) + x * kLog2eTail;
  float e = exp2_fast(t_hi);
  e = fmaf(e, t_lo * kLn2, e);
  const float s = e * rcp_fast(2.0f + e);
  const float s2 = s * s;
  float q = 1.0f / 13.0f;
  q = fmaf(q, s2, 1.0f / 11.0f);
  q = fmaf(q, s2, 1.0f / 9.0f);
  q = fmaf(q, s2, 1.0f / 7.0f);
  q = fmaf(q, s2, 1.0f / 5.0f);
  q = fmaf(q, s2, 1.0f / 3.0f);
  q = fmaf(q, s2, 1.0f);
  const float l = 2.0f * s * q;
  const float r = fmaxf(u, 0.0f) + l;
  return u != u ? u : r;
}

// ZOH input scale expm1(Delta a) / a from Abar = 2^t, t = Delta a log2(e), ia = 1 / a.
// fma(Abar, ia, -ia) = (Abar - 1) / a loses relative accuracy as |Delta a| shrinks: Abar carries an
// absolute rounding error of about 2^-24, so (Abar - 1) is off by about 6e-8 / |Delta a| relative.
// That is far inside the bf16 tolerance but not the float32 one, so with ACCURATE (float32 I/O)
// |Delta a| < 1/16 takes the series Delta (1 + z/2 + z^2/6 + z^3/24), z = Delta a = t ln 2, whose
// truncation error is below z^4 / 120 < 1.3e-7 relative; above it the fma form is within 2e-6.
// Base-2 exponent bound of the series: |t| < kZohSeriesT, i.e. |z| < 1/16.
constexpr float kZohSeriesT = 0.0625f / 0.6931471805599453f;

template <bool ACCURATE>
__device__ __forceinline__ float zoh_input_scale(float abar, float t, float dt, float ia) {
  const float s = fmaf(abar, ia, -ia);
  if constexpr (!ACCURATE) {
    return s;
  } else {
    constexpr float kLn2 = 0.6931471805599453f;
    constexpr float c1 = kLn2 / 2.0f;                       // ln2 / 2!
    constexpr float c2 = kLn2 * kLn2 / 6.0f;                // ln2^2 / 3!
    constexpr float c3 = kLn2 * kLn2 * kLn2 / 24.0f;        // ln2^3 / 4!
    constexpr float kSmallT = kZohSeriesT;
    float q = fmaf(t, c3, c2);
    q = fmaf(q, t, c1);
    const float ser = fmaf(dt * t, q, dt);
    return fabsf(t) < kSmallT ? ser : s;
  }
}

// Element loads/stores of the per-token tensors in either storage type.
template <typename T> struct IoTraits;

template <> struct IoTraits<float> {
  __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
  // one element's raw bits (conversion deferred so the load can stay in flight)
  __device__ __forceinline__ static uint32_t load_bits(const float* p, int64_t i) {
    return __float_as_uint(p[i]);
  }
  __device__ __forceinline__ static float from_bits(uint32_t v) { return __uint_as_float(v); }
  __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
  // four consecutive elements (16-byte aligned)
  __device__ __forceinline__ static void load4(const float* p, int64_t i, float out[4]) {
    float4 v = *reinterpret_cast<const float4*>(p + i);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
  __device__ __forceinline__ static void store4(float* p, int64_t i, const float v[4]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v[0], v[1], v[2], v[3]);
  }
  using raw4 = uint4;
  __device__ __forceinline__ static raw4 load4_raw(const float* p, int64_t i) {
    return *reinterpret_cast<const uint4*>(p + i);
  }
  __device__ __forceinline__ static void unpack4(raw4 r, float out[4]) {
    out[0] = __uint_as_float(r.x); out[1] = __uint_as_float(r.y);
    out[2] = __uint_as_float(r.z); out[3] = __uint_as_float(r.w);
  }
  __device__ __forceinline__ static raw4 zero4() { return make_uint4(0, 0, 0, 0); }
  // a 16-byte chunk: four elements
  __device__ __forceinline__ static void unpack_chunk(uint4 r, float out[4]) { unpack4(r, out); }
};

template <> struct IoTraits<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i].bits); }
  __device__ __forceinline__ static uint32_t load_bits(const bf16_t* p, int64_t i) { return p[i].bits; }
  __device__ __forceinline__ static float from_bits(uint32_t v) { return __uint_as_float(v << 16); }
  __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) { p[i].bits = f32_to_bf16(v); }
  using raw4 = uint2;
  // four consecutive elements (8-byte aligned)
  __device__ __forceinline__ static raw4 load4_raw(const bf16_t* p, int64_t i) {
    return *reinterpret_cast<const uint2*>(p + i);
  }
  __device__ __forceinline__ static void unpack4(raw4 r, float out[4]) {
    out[0] = bf16_lo(r.x); out[1] = bf16_hi(r.x); out[2] = bf16_lo(r.y); out[3] = bf16_hi(r.y);
  }
  __device__ __forceinline__ static void load4(const bf16_t* p, int64_t i, float out[4]) {
    unpack4(load4_raw(p, i), out);
  }
  __device__ __forceinline__ static void store4(bf16_t* p, int64_t i, const float v[4]) {
    const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(p + i) = make_uint2(lo, hi);
  }
  __device__ __forceinline__ static raw4 zero4() { return make_uint2(0, 0); }
  // a 16-byte chunk: eight elements
  __device__ __forceinline__ static void unpack_chunk(uint4 r, float out[8]) {
    out[0] = bf16_lo(r.x); out[1] = bf16_hi(r.x); out[2] = bf16_lo(r.y); out[3] = bf16_hi(r.y);
    out[4] = bf16_lo(r.z); out[5] = bf16_hi(r.z); out[6] = bf16_lo(r.w); out[7] = bf16_hi(r.w);
  }
};

// One element's raw bits / one element store in storage type io_t, through a descriptor.
__device__ __forceinline__ uint32_t buf_load_bits(Rsrc r, uint32_t off, float*) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_bits(Rsrc r, uint32_t off, bf16_t*) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(Rsrc r, uint32_t off, float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void buf_store(Rsrc r, uint32_t off, float v, bf16_t*) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
}

// Sum over the LPC lanes of a channel (aligned groups of 1, 2 or 4 consecutive lanes).
template <int LPC>
__device__ __forceinline__ float sum_channel_lanes(float v) {
  if constexpr (LPC >= 2) {
    // quad_perm [1, 0, 3, 2]: swap neighbouring lanes
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  }
  if constexpr (LPC >= 4) {
    // quad_perm [2, 3, 0, 1]: swap lane pairs
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
  }
  return v;
}

}  // namespace ssm

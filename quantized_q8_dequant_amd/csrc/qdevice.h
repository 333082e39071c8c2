// Device helpers shared by the gfx950 kernels: numeric conversions, the
// Q8_0 block quantiser, the integer half-block dot and wavefront reductions.
//
// The quantiser follows the Q8_0 encoder of the Fucina course page "Model
// files and quantization", section 11.7 (per 32 values: amax; d = amax/127;
// inv = d == 0 ? 0 : 1/d; q = round(v * inv) clamped to +-127; the stored
// scale is f16(d)) with round-half-to-even, the production rounding of
// section 11.10.  Divisions are IEEE (the build does not enable fast math),
// so the codes match a CPU encoder bit for bit on the same f32 input.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QDEV __device__ __forceinline__

namespace q8 {

constexpr int kWave = 64;

// ---- conversions -------------------------------------------------------------
QDEV float f16_bits_to_f32(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}
QDEV uint16_t f32_to_f16_bits(float x) {  // v_cvt_f16_f32: round to nearest even
  _Float16 h = (_Float16)x;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}
QDEV float f16_round(float x) { return (float)(_Float16)x; }

QDEV uint16_t f32_to_bf16_bits(float x) {  // round half to even on the dropped 16 bits
  uint32_t u = __float_as_uint(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
QDEV float bf16_bits_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
QDEV float bf16_round(float x) { return bf16_bits_to_f32(f32_to_bf16_bits(x)); }

// ---- global address space ----------------------------------------------------------
// A pointer read from a table in memory is generic to the compiler, which then
// emits flat loads.  Flat loads count against the LDS wait counter as well, so
// every later LDS wait would also drain the (slow) weight loads in flight.
// as_global() states that the pointer addresses global memory.
#define QGLOBAL __attribute__((address_space(1)))
template <typename T>
QDEV const QGLOBAL T* as_global(const T* p) {
  return (const QGLOBAL T*)(__UINTPTR_TYPE__)p;
}
template <typename T, typename U>
QDEV T ld_global(const QGLOBAL U* p) {  // a T-typed load at p
  return *reinterpret_cast<const QGLOBAL T*>(p);
}

// ---- cross-workgroup hand-off without cache-wide fences ---------------------------
// A device-wide fence writes back and invalidates the whole L2 of the XCD;
// thousands of workgroups doing that stall each other.  Data handed to
// another workgroup of the same launch is instead written and read with
// agent-scope atomic accesses (coherent across XCDs on their own), and the
// writer waits for its stores before it bumps the arrival counter.
template <typename T>
QDEV void st_coherent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
QDEV T ld_coherent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
QDEV void wait_memory() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);  // keep the compiler from moving accesses across
  __builtin_amdgcn_s_waitcnt(0);            // vmcnt = expcnt = lgkmcnt = 0
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
QDEV unsigned arrive(unsigned* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- wavefront reductions ----------------------------------------------------------
template <int WIDTH>
QDEV float wave_sum(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
  return v;
}
template <int WIDTH>
QDEV float wave_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WIDTH));
  return v;
}

template <int WIDTH>
QDEV double wave_sum_d(double v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, WIDTH);
  return v;
}
template <int WIDTH>
QDEV double wave_max_d(double v) {
#pragma unroll
  for (int o = WIDTH / 2; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o, WIDTH));
  return v;
}

// Sums of doubles over aligned groups of WIDTH lanes (WIDTH = 2..64) with DPP
// lane moves of the two 32-bit halves: quad permutes, the row mirrors and the
// GFX9 row broadcasts, a few cycles per step instead of an LDS-permute round
// trip.  The group's total is valid in its LAST lane (other lanes hold
// partial sums).
// (lanes of rows outside ROW_MASK receive `old`)
template <int CTRL, int ROW_MASK = 0xF>
QDEV double dpp_move_d(double v, double old = 0.0) {
  const int lo = __builtin_amdgcn_update_dpp(__double2loint(old), __double2loint(v), CTRL, ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(__double2hiint(old), __double2hiint(v), CTRL, ROW_MASK, 0xF, false);
  return __hiloint2double(hi, lo);
}
template <int WIDTH>
QDEV double group_sum_d(double v) {
  static_assert(WIDTH == 1 || WIDTH == 2 || WIDTH == 4 || WIDTH == 8 || WIDTH == 16 || WIDTH == 32 || WIDTH == 64,
                "group width");
  if (WIDTH >= 2) v += dpp_move_d<0xB1>(v);        // quad_perm [1,0,3,2]
  if (WIDTH >= 4) v += dpp_move_d<0x4E>(v);        // quad_perm [2,3,0,1]
  if (WIDTH >= 8) v += dpp_move_d<0x141>(v);       // row_half_mirror
  if (WIDTH >= 16) v += dpp_move_d<0x140>(v);      // row_mirror
  if (WIDTH >= 32) v += dpp_move_d<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  if (WIDTH >= 64) v += dpp_move_d<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
QDEV double bcast_last_d(double v) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(v), kWave - 1);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(v), kWave - 1);
  return __hiloint2double(hi, lo);
}
// The wavefront's total / maximum in every lane.
QDEV double wave_total_d(double v) { return bcast_last_d(group_sum_d<kWave>(v)); }
QDEV double wave_max_all_d(double v) {
  v = fmax(v, dpp_move_d<0xB1>(v));
  v = fmax(v, dpp_move_d<0x4E>(v));
  v = fmax(v, dpp_move_d<0x141>(v));
  v = fmax(v, dpp_move_d<0x140>(v));
  v = fmax(v, dpp_move_d<0x142, 0xA>(v, -INFINITY));
  v = fmax(v, dpp_move_d<0x143, 0xC>(v, -INFINITY));
  return bcast_last_d(v);
}

// Block-wide sum of one double per thread (blockDim.x == NT, NT % 64 == 0),
// without the trailing barrier: the caller passes another barrier before
// s_red is written again.  Same summation order as block_sum_d.
template <int NT>
QDEV double block_sum_d_open(double v, double* s_red) {
  v = group_sum_d<kWave>(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == kWave - 1) s_red[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += s_red[i];
  return t;
}

// The maximum over aligned groups of WIDTH lanes (16 or 32), in every lane
// of the group.
template <int WIDTH>
QDEV double group_max_all_d(double v) {
  static_assert(WIDTH == 16 || WIDTH == 32, "group width");
  v = fmax(v, dpp_move_d<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmax(v, dpp_move_d<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmax(v, dpp_move_d<0x141>(v));  // row_half_mirror
  v = fmax(v, dpp_move_d<0x140>(v));  // row_mirror: every lane holds its row's maximum
  if (WIDTH == 32) v = fmax(v, __shfl_xor(v, 16));
  return v;
}

// Block-wide sum of one double per thread (blockDim.x == NT, NT % 64 == 0).
template <int NT>
QDEV double block_sum_d(double v, double* s_red) {
  v = group_sum_d<kWave>(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == kWave - 1) s_red[w] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += s_red[i];
  __syncthreads();
  return t;
}

// RMSNorm scale r = 1 / sqrt(mean(x^2) + eps) from the f64 sum of squares
// (each square is exact in f64), then y = f32((x * r) * w) evaluated in f64:
// the value rounded once to f32, as a reference computing in f64 would.
QDEV double rms_scale(double sumsq, int n, float eps) { return 1.0 / sqrt(sumsq / (double)n + (double)eps); }
QDEV float rms_apply(float x, double r, float w) {
#pragma clang fp contract(off)
  return (float)(((double)x * r) * (double)w);
}

// silu(g) * u in f64 from the f32 values of g and u, rounded once to f32.
QDEV float swiglu_f64(float g, float u) {
#pragma clang fp contract(off)
  const double gd = (double)g;
  return (float)((gd / (1.0 + exp(-gd))) * (double)u);
}

// Block-wide sum of one float per thread (blockDim.x == NT, NT % 64 == 0).
template <int NT>
QDEV float block_sum(float v, float* s_red) {
  v = wave_sum<kWave>(v);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) s_red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < NT / kWave; ++i) t += s_red[i];
  __syncthreads();
  return t;
}

// ---- Q8_0 quantiser ---------------------------------------------------------------
// One 32-block is held by 8 consecutive lanes, 4 values each (v[0..3] are
// block elements 4*(lane%8) .. +3).  Returns the 4 codes packed in an int
// (byte i = code of v[i]) and the f32 scale d through *d_out (every lane of
// the group gets the same d).
QDEV int quant4_group8(const float v[4], float* d_out) {
  float a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  // max over the 8 lanes (DPP: quad permutes, then the half-row mirror)
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false)));
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x141, 0xF, 0xF, false)));
  const float d = a / 127.0f;
  const float inv = d == 0.f ? 0.f : 1.0f / d;
  int packed = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float q = rintf(v[i] * inv);
    q = fminf(fmaxf(q, -127.f), 127.f);
    packed |= ((int)q & 0xFF) << (8 * i);
  }
  *d_out = d;
  return packed;
}

// ---- integer dot of one 32-value block ---------------------------------------------
// S = sum_{i<32} a_i * b_i over signed bytes, exact in int32 (|S| <= 32 * 127^2),
// from two 16-byte halves per operand: 8 x v_dot4 in one lane (no cross-lane
// step, so the result never depends on another lane's timing).
typedef int v4i __attribute__((ext_vector_type(4)));

QDEV int dot32_i8(const v4i a0, const v4i a1, const v4i b0, const v4i b1) {
  int s = __builtin_amdgcn_sdot4(a0.x, b0.x, 0, false);
  s = __builtin_amdgcn_sdot4(a0.y, b0.y, s, false);
  s = __builtin_amdgcn_sdot4(a0.z, b0.z, s, false);
  s = __builtin_amdgcn_sdot4(a0.w, b0.w, s, false);
  s = __builtin_amdgcn_sdot4(a1.x, b1.x, s, false);
  s = __builtin_amdgcn_sdot4(a1.y, b1.y, s, false);
  s = __builtin_amdgcn_sdot4(a1.z, b1.z, s, false);
  s = __builtin_amdgcn_sdot4(a1.w, b1.w, s, false);
  return s;
}

// RMSNorm over one head (HD values in LDS, rounded to f32 as a separate
// step) followed by the NeoX rotation of pairs (i, i + HD/2) by the angle
// whose f64 cos/sin are cs[i]/sn[i], each output evaluated in f64 and rounded
// once to f32; run by one wavefront ("A transformer from scratch", sections
// 12.3.2 and 12.3.4).
template <int HD>
QDEV void norm_rope_wave(float* x, const float* __restrict__ w, float eps, const double* __restrict__ cs,
                         const double* __restrict__ sn) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x % kWave;
  double ss = 0.0;
  for (int d = lane; d < HD; d += kWave) ss += (double)x[d] * (double)x[d];
  ss = wave_total_d(ss);
  const double r = rms_scale(ss, HD, eps);
  constexpr int H2 = HD / 2;
  for (int i = lane; i < H2; i += kWave) {
    const double a = (double)rms_apply(x[i], r, w[i]);
    const double b = (double)rms_apply(x[i + H2], r, w[i + H2]);
    const double c = cs[i], s = sn[i];
    x[i] = (float)(a * c - b * s);
    x[i + H2] = (float)(a * s + b * c);
  }
}

// The same with this lane's operands already in registers, so they can be
// loaded before the values arrive: weights w[lane] and w[lane + HD/2], and the
// cos/sin of pair `lane` (lanes >= HD/2 carry no pair).  Same arithmetic and
// summation order as norm_rope_wave.
template <int HD>
QDEV void norm_rope_wave_reg(float* x, float wlo, float whi, double c, double s, float eps) {
#pragma clang fp contract(off)
  static_assert(HD / 2 <= kWave, "one rotation pair per lane");
  const int lane = threadIdx.x % kWave;
  double ss = 0.0;
  for (int d = lane; d < HD; d += kWave) ss += (double)x[d] * (double)x[d];
  ss = wave_total_d(ss);
  const double r = rms_scale(ss, HD, eps);
  constexpr int H2 = HD / 2;
  if (lane < H2) {
    const double a = (double)rms_apply(x[lane], r, wlo);
    const double b = (double)rms_apply(x[lane + H2], r, whi);
    x[lane] = (float)(a * c - b * s);
    x[lane + H2] = (float)(a * s + b * c);
  }
}

}  // namespace q8

// Internal declarations shared by the libfa translation units: kernel
// parameter blocks, launchers and gfx950 device helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

enum class Elem { F32 = 0, F16 = 1, BF16 = 2 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int* kv_len;  // device [B] or nullptr
  int B, H, N, d;
  float scale;
  int causal;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;  // workspace: D_i = rowsum(dO * O), [B, H, N] fp32
  const int* kv_len;
  int B, H, N, d;
  float scale;
  int causal;
};

// Launchers return hipSuccess or the launch error. Arguments are validated
// by the caller.
hipError_t launch_fwd_mfma(const FwdArgs& a, Elem in, Elem out, hipStream_t s);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t s);
// Backward stages: D_i = rowsum(dO * O), then dK/dV, then dQ. The dK/dV and
// dQ stages read only the inputs, LSE and D, so they may run in any order.
enum class BwdStage { DSUM = 1, DKDV = 2, DQ = 4, ALL = 7 };
hipError_t launch_bwd_mfma(const BwdArgs& a, Elem t, int stages, hipStream_t s);
hipError_t launch_bwd_f32(const BwdArgs& a, int stages, hipStream_t s);

// ---------------------------------------------------------------------------
// Device helpers (gfx950).

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 16-bit element tags: the kernels move raw 16-bit words and only the MFMA
// and the fp32 <-> 16-bit conversions care which format they hold.
struct BF16 {
  static constexpr Elem kind = Elem::BF16;
};
struct F16 {
  static constexpr Elem kind = Elem::F16;
};

template <typename T>
struct Mfma;

// D(32x32, fp32) += A(32x16) * B(16x32). Lane l holds row/column l % 32 of
// its operand and the k-group l / 32; A and B map (k-group, element) to the
// reduction index the same way, so any consistent assignment of actual
// indices to those slots yields the same contraction.
template <>
struct Mfma<BF16> {
  __device__ static inline f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Round-to-nearest-even pack of two fp32 into two bf16 (lo = a).
  __device__ static inline uint32_t pack(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float to_f32(uint16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x << 16);
  }
};

template <>
struct Mfma<F16> {
  __device__ static inline f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static inline uint32_t pack(float a, float b) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 r = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, r);
  }
  __device__ static inline float to_f32(uint16_t x) {
    return (float)__builtin_bit_cast(_Float16, x);
  }
};

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ inline float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (l ^ 32): the other half of the wave.
__device__ inline float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

// Block index remap so that consecutive logical blocks run on the same XCD.
// Workgroups are dealt round-robin to the 8 XCDs; logical block
// x * per + i is placed on physical slot i * 8 + x. Blocks past the largest
// multiple of 8 keep their index.
__device__ inline int xcd_remap(int bid, int total) {
  const int nxcd = 8;
  const int per = total / nxcd;
  if (bid >= per * nxcd) return bid;
  return (bid % nxcd) * per + bid / nxcd;
}

}  // namespace fa

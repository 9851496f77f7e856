// Device helpers shared by the gfx950 kernels of the block-quantized library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <tuple>

#include "qmv_layout.h"

namespace qmv {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// IEEE binary16 bit pattern -> fp32 (v_cvt_f32_f16; fp16 subnormals are kept:
// the fp16 denormal mode is on for HIP kernels).
__device__ __forceinline__ float fp16_bits_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Two nibble-valued bytes (each 0..15) of `bytes4`, selected by `hi_word`
// (bytes 0,1 or bytes 2,3), converted to two exact bf16 integers.
//
// A byte holding q in [0, 15], read as an OCP fp8 e4m3 value, equals q * 2^-9
// exactly (0..7 are the subnormals m * 2^-9, 8..15 have exponent field 1 and
// value (8 + m) * 2^-9), so the gfx950 scaled fp8 -> bf16 conversion with a
// scale of 2^9 returns q itself. One instruction yields two exact quants.
template <bool HI_WORD>
__device__ __forceinline__ bf16x2 nibbles_to_bf16x2(uint32_t bytes4) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(bytes4, 512.0f, HI_WORD);
}

// Lane permutation within DPP rows of 16 lanes (CTRL is a DPP control code).
template <int CTRL>
__device__ __forceinline__ float dpp_shuffle(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 16 lanes (one DPP row), left in every lane of
// the group. Each butterfly step adds a commutative pair, so all 16 lanes end
// with bit-identical values.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_shuffle<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_shuffle<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_shuffle<0x141>(v);  // row_half_mirror: quad 0 <-> quad 1 within each half row
  v += dpp_shuffle<0x140>(v);  // row_mirror: half row 0 <-> half row 1
  return v;
}

__device__ __forceinline__ float row8_sum(float v) {
  v += dpp_shuffle<0xB1>(v);
  v += dpp_shuffle<0x4E>(v);
  v += dpp_shuffle<0x141>(v);
  return v;
}

__device__ __forceinline__ float row4_sum(float v) {
  v += dpp_shuffle<0xB1>(v);
  v += dpp_shuffle<0x4E>(v);
  return v;
}

// Sum over aligned groups of G lanes (G in {4, 8, 16, 32, 64}); every lane of a
// group ends with the same bits (each step adds a commutative pair).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
  if constexpr (G == 4) return row4_sum(v);
  else if constexpr (G == 8) return row8_sum(v);
  else {
    v = row16_sum(v);
    if constexpr (G >= 32) v += __shfl_xor(v, 16);
    if constexpr (G == 64) v += __shfl_xor(v, 32);
    return v;
  }
}

// Record a HIP failure for qmv_last_error() (thread-local text kept by the ABI layer).
void set_error_detail(const char *what, int hip_code, const char *hip_text);

// Host-side launch that reports the launch status itself (QMV_OK = 0 or
// QMV_ERR_HIP = -8) instead of reading the thread's sticky last-error state.
template <typename... Params, typename... Args>
inline int launch_kernel(const char *name, void (*kernel)(Params...), dim3 grid, dim3 block, size_t lds,
                         hipStream_t stream, Args... args) {
  static_assert(sizeof...(Params) == sizeof...(Args), "argument count");
  auto typed = std::make_tuple(static_cast<Params>(args)...);
  void *argv[sizeof...(Params)];
  std::apply([&argv](auto &...a) {
    int i = 0;
    ((argv[i++] = static_cast<void *>(&a)), ...);
  }, typed);
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, lds, stream);
  if (e != hipSuccess) {
    set_error_detail(name, (int)e, hipGetErrorString(e));
    return -8;
  }
  return 0;
}

// Dynamic-LDS sizes already granted to one kernel, per device (the attribute
// belongs to the kernel on the device that is current when it is set).
struct LdsGrant {
  static constexpr int kDevices = 64;
  std::atomic<size_t> dev[kDevices] = {};
};

// Allow `bytes` of dynamic LDS for `kernel` on the current device (needed above
// 64 KiB). The largest value granted so far is remembered per call site and
// device, so the attribute is set once per size increase rather than on every
// launch. This cache never changes what a kernel computes.
inline int allow_dynamic_lds(const void *kernel, size_t bytes, LdsGrant &granted, const char *name) {
  if (bytes <= 65536) return 0;
  int d = 0;
  hipError_t e = hipGetDevice(&d);
  if (e == hipSuccess && (d < 0 || d >= LdsGrant::kDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    set_error_detail(name, (int)e, hipGetErrorString(e));
    return -8;
  }
  std::atomic<size_t> &g = granted.dev[d];
  if (bytes <= g.load(std::memory_order_relaxed)) return 0;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) {
    set_error_detail(name, (int)e, hipGetErrorString(e));
    return -8;
  }
  size_t cur = g.load(std::memory_order_relaxed);
  while (cur < bytes && !g.compare_exchange_weak(cur, bytes)) {
  }
  return 0;
}

}  // namespace qmv

// Device helpers shared by the forward and backward kernels (gfx950 / CDNA4):
// vector types, the 32x32x16 MFMA for fp16 and bf16, cross-half reductions, the
// transposing LDS read, buffer resources with zero fill past the end, direct
// memory-to-LDS loads, the XOR swizzle of K/V-style tiles in LDS, and the host-side
// launch helper.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.6931471805599453f;

// Launches kernel(arg) with `grid` workgroups of `block` threads on `stream` and
// returns the status of this launch alone. (hipGetLastError after a <<<>>> launch
// would also return, and clear, an error that an earlier, unrelated HIP call of the
// caller's thread left pending: a successful launch would then be reported as failed,
// and the caller's own error lost.)
template <class P>
inline hipError_t launch_kernel(void (*kernel)(P), int64_t grid, int block, hipStream_t stream, P arg) {
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3((unsigned)grid), dim3((unsigned)block), args,
                         0, stream);
}

template <bool BF16> struct Elem;
template <> struct Elem<false> { using vec8 = f16x8; };
template <> struct Elem<true> { using vec8 = bf16x8; };

template <bool BF16>
__device__ __forceinline__ f32x16 mfma_32x32x16(i16x8 a, i16x8 b, f32x16 c) {
  using V = typename Elem<BF16>::vec8;
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(V, a), __builtin_bit_cast(V, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(V, a), __builtin_bit_cast(V, b), c, 0, 0, 0);
}

// Reductions across the two 32-lane halves of a wave. v_permlane32_swap with the
// same register as both operands leaves the low half's value in every lane of r[0]
// and the high half's value in every lane of r[1].
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ i16x4 ds_read_tr16(const short* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) short*)lds_ptr));
}

// Buffer resource over [base, base + bytes): loads at offsets past the end return
// zeros, which pads the ragged last key/query tile without any branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ i16x8 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(i16x8, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}
// 16 bytes per lane straight from memory into LDS: lane l writes LDS bytes
// [lds + 16 l, lds + 16 l + 16) (lds is wave-uniform); out-of-range lanes write zeros.
// AUX: the cache-policy bits of the load (0: default; 2: non-temporal, for data read
// once).
template <int AUX = 0>
__device__ __forceinline__ void buffer_load16_to_lds(__amdgpu_buffer_rsrc_t r, short* lds, uint32_t voff,
                                                     uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) short*)lds), 16, voff, soff,
      0, AUX);
}

// K and V tiles sit in LDS without padding, as rows of D 16-bit elements whose
// 16-byte chunks are XOR-permuted per row: chunk c of row r is stored at chunk
// position c ^ swz(r). For both the 32-row K fragment reads (16 lanes x 16 B) and the
// transposing V reads (4 rows x 64 B per half wave) every access of a wave then
// touches distinct banks. swz has period 16 in r.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}

}  // namespace

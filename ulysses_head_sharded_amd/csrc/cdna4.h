// cdna4.h -- device helpers shared by the gfx950 attention kernels: operand
// types of the 32x32x16 bf16 MFMA, raw buffer resources, direct
// global->LDS loads, the transposing LDS read and the half-wave exchange.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ulys {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// dword 3 of a raw buffer resource (no swizzle, 32-bit data format) on gfx9
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }
// Reinterpret a whole vector.  Note: __builtin_bit_cast applied to one
// element of an ext_vector (bit_cast<float>(v[i])) is lowered by this
// compiler as a read of element 0 whatever i is; cast the whole vector and
// index the result instead.
__device__ __forceinline__ f32x4 as_f32x4(u32x4 x) { return __builtin_bit_cast(f32x4, x); }

// Raw buffer resource over a whole tensor: loads past num_bytes return 0 and
// stores past it are dropped, which handles ragged tails without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, num_bytes,
                                           kRsrcWord3);
}

// The value of x in the partner lane (l ^ 32) combined with max / sum.
__device__ __forceinline__ float xmax32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)sw[0]),
               __builtin_bit_cast(float, (uint32_t)sw[1]));
}
__device__ __forceinline__ float xsum32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)sw[0]) + __builtin_bit_cast(float, (uint32_t)sw[1]);
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// output lane 4a+e receives element e of the 8-byte reads of source lanes a,
// a+4, a+8, a+12.  When source lane s reads 4 elements at row r0 + s/4,
// column c0 + 4 (s%4) of a row-major tile, output lane L therefore holds
// rows r0 .. r0+3 of column c0 + L: four consecutive rows of one feature,
// i.e. one half of an MFMA operand taken straight from a row-major tile.
// The restrict qualifier gives the access alias scope, so the compiler does
// not make it wait for unrelated direct global->LDS loads.
__device__ __forceinline__ u32x2 lds_read_tr(const uint16_t* __restrict__ p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// One direct global->LDS load: every lane's 16 bytes at byte offset voff of
// the resource land at lds_dst + 16 * lane (out-of-range lanes write zeros).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_dst, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_dst,
                                           16, voff, 0, 0, 0);
}

}  // namespace ulys

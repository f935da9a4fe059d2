// device_common.h -- gfx950 (CDNA4) device helpers shared by the attention kernels.
//
// Vector types, the bf16/f16 element traits used by the MFMA paths (matrix
// instruction, packed conversion, two-element dot product, LDS transpose
// read), and small wave-level utilities.  Internal to libattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef float floatx2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define ATTN_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// Element traits for the two 16-bit input types.  `mma32` is
// D = A * B + C on the 32x32x16 matrix instruction; `mma16` the 16x16x32 one.
template <typename T>
struct Elem;

template <>
struct Elem<__bf16> {
  using x8 = bf16x8;
  using x2 = bf16x2;
  static __device__ __forceinline__ floatx16 mma32(u32x4 a, u32x4 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(x8, a),
                                                  __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mma16(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(x8, a),
                                                  __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  // Two floats -> two packed elements, round to nearest even.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    floatx2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, x2));
  }
  // c + a.lo * b.lo + a.hi * b.hi with float32 accumulation.
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(x2, a), __builtin_bit_cast(x2, b),
                                           c, false);
  }
  static constexpr uint32_t kOnePair = 0x3f803f80u;  // (1.0, 1.0)
  // the low 16 bits of h as a bf16 value
  static __device__ __forceinline__ float to_float(uint32_t h) { return __builtin_bit_cast(float, h << 16); }
  static __device__ __forceinline__ float lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
  static __device__ __forceinline__ float hi(uint32_t v) {
    return __builtin_bit_cast(float, v & 0xffff0000u);
  }
};

template <>
struct Elem<_Float16> {
  using x8 = f16x8;
  using x2 = f16x2;
  static __device__ __forceinline__ floatx16 mma32(u32x4 a, u32x4 b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(x8, a),
                                                 __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ floatx4 mma16(u32x4 a, u32x4 b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(x8, a),
                                                 __builtin_bit_cast(x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    floatx2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, x2));
  }
  static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(x2, a), __builtin_bit_cast(x2, b), c, false);
  }
  static constexpr uint32_t kOnePair = 0x3c003c00u;  // (1.0, 1.0)
  // the low 16 bits of h as an f16 value
  static __device__ __forceinline__ float to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)h);
  }
  static __device__ __forceinline__ float lo(uint32_t v) {
    return (float)__builtin_bit_cast(f16x2, v)[0];
  }
  static __device__ __forceinline__ float hi(uint32_t v) {
    return (float)__builtin_bit_cast(f16x2, v)[1];
  }
};

// LDS transpose read of 16-bit data (ds_read_b64_tr_b16).  Within each group
// of 16 lanes, lane 4*r + p supplies the address of 4 consecutive elements
// (piece p of row r of a 4 x 16 block); afterwards lane i of the group holds
// column i of that block: (row0[i], row1[i], row2[i], row3[i]).
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_addr) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((ATTN_LDS i16x4*)(lds_addr));
  return __builtin_bit_cast(u32x2, v);
}

// Full max / sum over the two 32-lane halves of a wave: lane l and lane l^32
// exchange values with one cross-half swap.
__device__ __forceinline__ float halves_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]),
                         __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

// True in every lane if `pred` holds in any active lane of the wave.
__device__ __forceinline__ bool wave_any(bool pred) {
  return __builtin_amdgcn_ballot_w64(pred) != 0;
}

__device__ __forceinline__ u32x4 zero_u32x4() { return u32x4{0u, 0u, 0u, 0u}; }

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Raw buffer resource over [base, base + bytes): loads past the end read 0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long long bytes) {
  const int n = bytes > 0x7fffffffLL ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// Same with a 32-bit size (clamped below at 0), for ranges known to be < 2 GiB:
// the clamp stays in scalar arithmetic.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes < 0 ? 0 : bytes, 0x00020000);
}

// Cache-policy operand of the buffer loads: non-temporal (streamed data that
// is read once; the caches do not keep it at the expense of reused lines).
constexpr int kLoadStream = 2;

// Asynchronous copy of 16 bytes per lane from a buffer to LDS: lane l's bytes
// land at lds_base + 16 * l (lds_base must be the same in every lane).
// POLICY is the cache-policy operand (0: default, kLoadStream: read once).
template <int POLICY = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void* lds_base, int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (ATTN_LDS void*)lds_base, 16, byte_off, 0, 0, POLICY);
}

// Waits until this wave's outstanding vector-memory loads (including the
// buffer-to-LDS copies above) have completed.  Issued through the builtin so
// that the compiler's own wait insertion knows every earlier load is done
// (GFX9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15 = no wait on the other two).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

}  // namespace attn

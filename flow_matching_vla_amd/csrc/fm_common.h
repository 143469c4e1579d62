// Internal definitions shared by the HIP kernels of the denoise loop (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

namespace fm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------------------
// MFMA traits. Both element types move operands as one 16-byte fragment per lane per
// k-chunk: lane l holds the (l / 16)-th run of VEC consecutive k of row (A) or column (B)
// (l % 16). The bf16 chunk is one v_mfma_f32_16x16x32_bf16; the fp32 chunk is four
// v_mfma_f32_16x16x4_f32, element j of every lane feeding instruction j. A and B use the
// same k assignment, so every chunk computes the exact 16x16 block product. The 16x16
// fp32 result: lane l, element i holds row 4 * (l / 16) + i, column l % 16.
// ---------------------------------------------------------------------------------------
template <typename T> struct Mma;

template <> struct Mma<bf16> {
  static constexpr int VEC = 8;   // elements per 16-byte fragment
  static constexpr int KC = 32;   // k covered by one fragment pair
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<float> {
  static constexpr int VEC = 4;
  static constexpr int KC = 16;
  typedef f32x4 frag;
  static __device__ __forceinline__ f32x4 mma(const frag& a, const frag& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
  }
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE

// 16 bytes of T as a native vector (kept in registers; no struct-with-array)
typedef uint32_t V16 __attribute__((ext_vector_type(4)));

template <typename T> __device__ __forceinline__ void unpack(const V16& v, float* out);
template <> __device__ __forceinline__ void unpack<float>(const V16& v, float* out) {
  out[0] = __uint_as_float(v[0]); out[1] = __uint_as_float(v[1]);
  out[2] = __uint_as_float(v[2]); out[3] = __uint_as_float(v[3]);
}
template <> __device__ __forceinline__ void unpack<bf16>(const V16& v, float* out) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    out[2 * j] = __uint_as_float(v[j] << 16);
    out[2 * j + 1] = __uint_as_float(v[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ uint32_t bf16_bits_rne(float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (bf16)x); }
template <typename T> __device__ __forceinline__ V16 pack(const float* in);
template <> __device__ __forceinline__ V16 pack<float>(const float* in) {
  V16 v;
  v[0] = __float_as_uint(in[0]); v[1] = __float_as_uint(in[1]);
  v[2] = __float_as_uint(in[2]); v[3] = __float_as_uint(in[3]);
  return v;
}
template <> __device__ __forceinline__ V16 pack<bf16>(const float* in) {
  V16 v;
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = bf16_bits_rne(in[2 * j]) | (bf16_bits_rne(in[2 * j + 1]) << 16);
  return v;
}
__device__ __forceinline__ V16 vzero() { return V16{0u, 0u, 0u, 0u}; }

// Eight FP8 E4M3 codes (two words, k order) to the bf16 MFMA operand, exactly (a row's
// power-of-two scale is applied to the sums instead).
__device__ __forceinline__ V16 fp8x8_bf16(uint32_t w0, uint32_t w1) {
  return V16{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, false)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.f, true)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, false)),
             __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.f, true))};
}

// GELU, tanh form: 0.5 x (1 + tanh z) with z = sqrt(2/pi) (x + 0.044715 x^3), evaluated as
// x / (1 + e^(-2z)) (the same function: 0.5 (1 + tanh z) = 1 / (1 + e^(-2z))), one
// exponential and one division instead of a full tanh.
__device__ __forceinline__ float gelu_tanh(float x) {
  const float c2 = 1.5957691216057308f;  // 2 sqrt(2 / pi)
  return x / (1.0f + __expf(-c2 * (x + 0.044715f * x * x * x)));
}
__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// Sixteen zero bytes to read in place of an absent optional operand: kernels load from
// (p ? p + i : g_zeros) unconditionally, because a load under a branch, even a uniform
// one, is waited on before the branch rejoins and so costs a memory round trip of its own.
static __device__ __attribute__((aligned(16))) float g_zeros[4] = {0.f, 0.f, 0.f, 0.f};

// Device-scope (sc1) scalar accesses for data exchanged between workgroups of one kernel.
__device__ __forceinline__ void st_dev1(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev1(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Buffer resources (raw, stride 0): loads at a byte offset at or past `bytes` return zeros
// and touch no memory, so edge tiles need neither clamped addresses nor selects.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ V16 bload16(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
// Raw buffer descriptor as four SGPRs (base, stride 0, byte extent, gfx9 format word).
__device__ __forceinline__ V16 make_desc(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)p;
  return V16{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// LDS byte address of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}
// 16 bytes per lane copied from a buffer straight into LDS: lane l's bytes land at
// lds + 16 l (lds wave-uniform). Issued as inline asm so the compiler does not treat every
// later LDS read as dependent on it; callers order it with explicit vmcnt waits and
// barriers. M0 (the LDS base of the copy) is saved and restored around it.
__device__ __forceinline__ void dma16_lds(const V16& desc, uint32_t lds, uint32_t off) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "buffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds), "v"(off), "s"(desc)
      : "memory");
}

// Storage slot of key j in a transposed V plane ([d][key]). For bf16 each aligned run of 32
// keys is permuted so that the eight keys one lane feeds to the P.V product, keys
// 16 h + 4 q + r (h = 0, 1; r = 0..3) for lane group q, sit contiguously at 8 q + 4 h + r;
// the attention kernel produces P in exactly that order from its transposed score tile.
// fp32 fragments hold four keys, 4 q + r, already contiguous.
template <typename T> __host__ __device__ __forceinline__ int vt_slot(int j);
template <> __host__ __device__ __forceinline__ int vt_slot<float>(int j) { return j; }
template <> __host__ __device__ __forceinline__ int vt_slot<bf16>(int j) {
  return (j & ~31) | (((j >> 2) & 3) << 3) | (((j >> 4) & 1) << 2) | (j & 3);
}

// Data-parallel-primitive (DPP) lane moves: VALU operands read from another lane of the
// same 16-lane row, no LDS traffic. quad_perm [1,0,3,2] / [2,3,0,1] swap neighbours and
// pairs within a quad; the half-row mirror maps lane i to 7 - i within each 8 lanes and
// the row mirror i to 15 - i.
template <int CTRL> __device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
// Sum over each aligned group of G consecutive lanes (G = 1, 2, 4, 8 or 16); every lane
// of the group gets the same total (each step adds values that the partners hold equally).
template <int G> __device__ __forceinline__ float group_sum(float x) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "group size");
  if constexpr (G >= 2) x += dpp_mov<kDppXor1>(x);
  if constexpr (G >= 4) x += dpp_mov<kDppXor2>(x);
  if constexpr (G >= 8) x += dpp_mov<kDppHalfMirror>(x);
  if constexpr (G >= 16) x += dpp_mov<kDppMirror>(x);
  return x;
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the four lane groups that hold one
// column of a 16x16 MFMA result), with VALU lane swaps instead of LDS permutes. Swapping a
// value with itself across 16-lane rows gives the pair (row 2i, row 2i+1) in every lane of
// both rows; across 32-lane halves, the pair (low half, high half). The result is the same
// in all four lanes.
__device__ __forceinline__ float group4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// The XCD (accelerator complex die) this wave runs on, from the hardware register.
__device__ __forceinline__ uint32_t hw_xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID, 0, 4)" : "=s"(v));
  return v;
}
// Logical item of a workgroup when each XCD must run one contiguous range of the launch's
// items (so that the items of a range exchange data through that XCD's L2): the range of the XCD
// the workgroup actually runs on, and its place in that range from blockIdx.x / 8. The dispatcher
// deals a launch's workgroups round-robin over the 8 XCDs of a whole-GPU partition, but the first
// workgroup does not always go to XCD 0 (a launch queued right behind another can start where
// that one stopped): each XCD then still receives exactly one residue class of blockIdx.x mod 8,
// so this map is a bijection onto [0, nblocks) for any starting XCD. nblocks is a multiple of 8.
__device__ __forceinline__ int xcd_range_item(int nblocks) {
  return (int)hw_xcc_id() * (nblocks >> 3) + (int)(blockIdx.x >> 3);
}

// Map a linear workgroup id so that consecutive logical ids land on the same XCD:
// the hardware deals workgroups round-robin over the 8 XCDs.
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  const int nx = 8;
  if (nblocks < nx || nblocks % nx != 0) return bid;
  return (bid % nx) * (nblocks / nx) + bid / nx;
}

}  // namespace fm

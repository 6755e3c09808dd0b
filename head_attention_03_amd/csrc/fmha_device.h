// Device primitives and host helpers shared by the attention kernels of libfmha (gfx950).
// Internal to the library: not part of the C ABI in include/fmha.h.
#ifndef FMHA_DEVICE_H_
#define FMHA_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace fmha {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kRescaleThreshold = 8.0f;  // log2 units: raise the running max only past 2^8
constexpr uint32_t kRsrcWord3 = 0x00020000u;  // gfx9 buffer descriptor: raw 32-bit dwords

enum : int { kF16 = 0, kBF16 = 1, kF8 = 2 };

// ------------------------------------------------------------------------------------
// device primitives
// ------------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) i32x4 lds_i32x4;
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, (int)kRsrcWord3);
}

// Same descriptor as raw SGPR words, for the inline-asm LDS-direct load below.
__device__ inline i32x4 make_rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  const i32x4 r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)a), __builtin_amdgcn_readfirstlane((int)(a >> 32)),
                   __builtin_amdgcn_readfirstlane((int)bytes), (int)kRsrcWord3};
  return r;
}

// 16 bytes per lane from a buffer straight into LDS at lds_addr + 16 * lane (lds_addr is
// wave-uniform).  Written as inline asm so the compiler does not track it: it would
// otherwise wait for these loads before LDS reads it cannot prove disjoint, which undoes the
// prefetch; the phase schedule waits for them explicitly.  No memory clobber: the LDS reads
// of the current stage may move across it (it only ever writes the other stage), while the
// volatile asm statements (loads, waits, barriers) keep their order.  M0 is saved and restored.
__device__ inline void lds_load16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  int saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(rsrc), "s"(lds_addr));
}

__device__ inline float wave_row_max(float x) {  // max of lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ inline float wave_row_sum(float x) {  // sum of lanes l and l^32
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x), __builtin_bit_cast(unsigned, x),
                                            false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Workgroup barrier for the phase schedule.  Unlike __syncthreads() it carries no release
// fence, which would also wait for the K/V loads still in flight for a later phase; the only
// ordering needed is that this wave's LDS reads have returned (lgkmcnt(0)) before another
// wave may overwrite the buffer, and the loads are waited for explicitly (vmcnt) where due.
__device__ inline void phase_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// s_waitcnt vmcnt(N)
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte chunk swizzle of a K/V/Q tile row j in LDS (CPR chunks per row), for the 64
// four-byte banks of the gfx950 LDS, which serve a b128 read 16 lanes at a time and a b64 read
// 32 lanes at a time.  Row j's chunks are XORed with a value of bits 0..3 of j only (so rows
// 16 apart share it): the 16 rows of a b128 group land on 16 distinct bank groups for the
// row-wise operand reads, and the 4 rows x 4 chunks of a 32-lane ds_read_b64_tr_b16 group
// cover all 64 banks for the transposed reads.
template <int CPR>
__device__ inline int swz(int j) {
  if constexpr (CPR >= 16) return (((j & 3) << 2) | ((j >> 2) & 3)) & (CPR - 1);
  if constexpr (CPR == 8) return (((j >> 1) & 1) << 2) | ((j >> 2) & 3);
  return (j >> 2) & 3;
}

template <int DT>
struct Elem;
template <>
struct Elem<kBF16> {
  typedef bf16x8 frag;
  __device__ static inline uint32_t pack(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  // the two packed values as fp32 (exact)
  __device__ static inline float lo(uint32_t pk) { return __builtin_bit_cast(float, pk << 16); }
  __device__ static inline float hi(uint32_t pk) { return __builtin_bit_cast(float, pk & 0xFFFF0000u); }
  __device__ static inline f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                  0, 0, 0);
  }
};
template <>
struct Elem<kF16> {
  typedef f16x8 frag;
  __device__ static inline uint32_t pack(float a, float b) {
    f16x2 v = {(_Float16)a, (_Float16)b};  // v_cvt_pk_f16_f32, round to nearest even
    return __builtin_bit_cast(uint32_t, v);
  }
  // the two packed values as fp32 (exact)
  __device__ static inline float lo(uint32_t pk) { return (float)__builtin_bit_cast(f16x2, pk)[0]; }
  __device__ static inline float hi(uint32_t pk) { return (float)__builtin_bit_cast(f16x2, pk)[1]; }
  __device__ static inline f32x16 mma(i32x4 a, i32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                 0, 0);
  }
};

// fp8 e4m3 (OCP e4m3fn): S^T and O^T on the 32x32x64 f8f6f4 MFMA, unit block scales
// (E8M0 127 = 2^0) since the per-tensor scales are folded into scale and o_scale.
__device__ inline f32x16 mma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// four fp32 values -> four e4m3 bytes (round to nearest even; inputs within +-448)
__device__ inline uint32_t pack_f8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
template <int I>
__device__ inline float f8_byte(uint32_t w) { return __builtin_amdgcn_cvt_f32_fp8((int)w, I); }

// 16-byte chunk swizzle of an 8-bit K/V tile row j in LDS (CPR chunks per row, P = 256 / row
// bytes rows per 256-byte bank window).  The 16 rows of a b128 K read land in 16 distinct
// chunk slots of the bank window, and so do the 8 rows x 2 chunks of a transposed 8-bit V read.
template <int CPR>
__device__ inline int swz8(int j) {
  constexpr int P = 256 / (16 * CPR);
  return 2 * ((j / P) % (CPR / 2)) + ((j >> 3) & 1);
}

// ------------------------------------------------------------------------------------
// host helpers
// ------------------------------------------------------------------------------------
// compute units of the current device (cached per device; 0 if the query fails)
inline int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev >= 0 && dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace fmha

#endif  // FMHA_DEVICE_H_

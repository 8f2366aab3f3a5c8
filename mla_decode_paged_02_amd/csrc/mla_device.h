// Device-side building blocks shared by the MLA kernels (gfx950 / CDNA4 only).
//
// Layout facts the kernels rely on (checked on the device by an in-bounds probe of the
// builtins' lane layouts):
//   * v_mfma_f32_16x16x32_bf16: lane l = 16*g + n holds A[n][8g..8g+7], B[8g..8g+7][n]
//     and returns D[4g + i][n], i = 0..3.
//   * ds_read_b64_tr_b16: within each 16-lane group, lane 16g + 4r + q supplies four
//     16-bit values M[r][4q..4q+3]; lane 16g + j receives M[0..3][j].
//   * global_load_lds_dwordx4: lane l's 16 bytes land at LDS base + 16*l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;

#define MLA_LDS __attribute__((address_space(3)))

constexpr int kHeadDim = 576;    // latent 512 + rope 64
constexpr int kLatentDim = 512;
constexpr int kRowBytes = 1152;  // one bf16 cache row
constexpr int kRowChunks = 72;   // 16-byte chunks per cache row
constexpr int kStageKeys = 32;   // keys per pipeline stage
constexpr int kTileKeys = 32;    // keys per scheduling tile (work-split granularity): one stage
constexpr int kStageBytes = kStageKeys * kRowBytes;  // 36864
constexpr int kDmaPerStage = kStageBytes / 1024;     // 36 wave-wide 16-byte loads
constexpr int kNumBuf = 4;       // stage buffers in LDS
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag behind

enum : uint32_t {
  kErrPageId = 1u,
  kErrSparseIndex = 2u,
  kErrOffsets = 4u,
  kErrCacheLen = 8u,
};

enum : int { kMaskNull = 0, kMaskCausal = 1, kMaskSliding = 2 };

// ---------------------------------------------------------------------------------------
// LDS tile layout: stage rows of 72 16-byte chunks (1152 bytes); chunk c of row r is
// stored at chunk c ^ s(r) with s(r) in 0..7, a permutation inside each aligned group of 8
// chunks.  s is linear in the row bits r0..r4:
//   s = (r1 ^ r3) << 2 | (r0 ^ r1 ^ r4) << 1 | r1,
// chosen so that the score reads (16-byte reads of the 16 rows 8a + b + 4u, b < 4) and the
// transposing value reads (8-byte reads of the rows 8g + b + 4u) meet each bank once per
// cycle whether the LDS serves them as 64 banks with consecutive rows half a bank window
// apart or as 128-byte windows in which every row starts at the same bank, and for each
// lane grouping of the 16-byte reads that agrees with the measured conflict counts
// (SQ_LDS_BANK_CONFLICT).  Because s leaves bits 3 and up of the chunk index alone, every
// read of a stage is one per-lane base plus a compile-time offset.  The map is an
// involution.
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int swz_mask(int row) {
  return ((((row >> 1) ^ (row >> 3)) & 1) << 2) | (((row ^ (row >> 1) ^ (row >> 4)) & 1) << 1) | ((row >> 1) & 1);
}
__device__ __forceinline__ int swz_chunk(int row, int c) { return c ^ swz_mask(row); }

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left unconstrained (gfx9 encoding).  n is
// clamped to the counter's 6-bit range; waiting for fewer outstanding loads than asked
// is always safe.
template <int N>
__device__ __forceinline__ void vm_wait_imm() {
  constexpr int n = N > 63 ? 63 : N;
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void vm_wait(int n) {
  switch (n) {
#define MLA_VMW(k) case k: vm_wait_imm<k>(); break;
    MLA_VMW(1) MLA_VMW(2) MLA_VMW(3) MLA_VMW(4) MLA_VMW(5) MLA_VMW(6) MLA_VMW(7) MLA_VMW(8)
    MLA_VMW(9) MLA_VMW(10) MLA_VMW(11) MLA_VMW(12) MLA_VMW(13) MLA_VMW(14) MLA_VMW(15)
    MLA_VMW(16) MLA_VMW(17) MLA_VMW(18) MLA_VMW(19) MLA_VMW(20) MLA_VMW(21) MLA_VMW(22)
    MLA_VMW(23) MLA_VMW(24) MLA_VMW(25) MLA_VMW(26) MLA_VMW(27) MLA_VMW(28) MLA_VMW(29)
    MLA_VMW(30) MLA_VMW(31) MLA_VMW(32) MLA_VMW(33) MLA_VMW(34) MLA_VMW(35) MLA_VMW(36)
    MLA_VMW(37) MLA_VMW(38) MLA_VMW(39) MLA_VMW(40) MLA_VMW(41) MLA_VMW(42) MLA_VMW(43)
    MLA_VMW(44) MLA_VMW(45) MLA_VMW(46) MLA_VMW(47) MLA_VMW(48) MLA_VMW(49) MLA_VMW(50)
    MLA_VMW(51) MLA_VMW(52) MLA_VMW(53) MLA_VMW(54) MLA_VMW(55) MLA_VMW(56) MLA_VMW(57)
    MLA_VMW(58) MLA_VMW(59) MLA_VMW(60) MLA_VMW(61) MLA_VMW(62) MLA_VMW(63)
#undef MLA_VMW
    default:
      if (n >= 64) vm_wait_imm<63>(); else vm_wait_imm<0>();
      break;
  }
}
__device__ __forceinline__ void lgkm_wait0() { __builtin_amdgcn_s_waitcnt((63 & 15) | (3 << 14) | (7 << 4)); }
__device__ __forceinline__ void all_wait0() { __builtin_amdgcn_s_waitcnt(0); }

// Barrier that also keeps the compiler from moving memory accesses across it, without
// the hardware fence __syncthreads adds (the caller states the waits it needs).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Direct global->LDS load of 16 bytes per lane (lane l lands at dst + 16*l).  Issued as
// inline assembly so that the compiler does not treat every later LDS read as a possible
// alias of it (it would then wait for all outstanding loads); the kernels state the
// vmcnt waits these loads need themselves.  m0 must be set one wait state before use.
// m0 is named as clobbered so that nothing the compiler keeps in it is assumed to survive.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* src, MLA_LDS void* dst_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}

// 4 bytes per lane: lane l's dword lands at dst_wave_base + 4 l.
__device__ __forceinline__ void dma4(const void* src, MLA_LDS void* dst_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}

// The same load with the source split into a wave-uniform 64-bit base (scalar registers)
// and a per-lane 32-bit byte offset, which needs no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void dma16_base(const void* base, uint32_t off, MLA_LDS void* dst_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
// Streaming forms of dma16 / dma16_base for data read once (non-temporal cache policy).
__device__ __forceinline__ void dma16_nt(const void* src, MLA_LDS void* dst_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(lds), "v"(src)
               : "memory", "m0");
}
__device__ __forceinline__ void dma16_base_nt(const void* base, uint32_t off, MLA_LDS void* dst_wave_base) {
  const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(lds), "v"(off), "s"(base)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 ds_read_tr16(const MLA_LDS void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS bf16x4*)p);
}

// Load through the constant address space: a wave-uniform address becomes a scalar
// (SMEM) load, counted by lgkmcnt instead of vmcnt.  Only for data the kernel never
// writes (page tables, offsets, lengths, index lists).
template <typename T>
__device__ __forceinline__ T ld_const(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Max / sum over the four lanes l, l^16, l^32, l^48, left in all four.  The lane swaps are
// VALU instructions of gfx950: with both operands equal, permlane32_swap returns the lower
// and the upper half of the wave in each half, permlane16_swap the even and the odd rows.
__device__ __forceinline__ float xor16_32_pair_max(float v, bool sum) {
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto h = __builtin_amdgcn_permlane32_swap(b, b, false, false);
  const float h0 = __builtin_bit_cast(float, (uint32_t)h[0]), h1 = __builtin_bit_cast(float, (uint32_t)h[1]);
  v = sum ? h0 + h1 : fmaxf(h0, h1);
  const uint32_t c = __builtin_bit_cast(uint32_t, v);
  const auto r = __builtin_amdgcn_permlane16_swap(c, c, false, false);
  const float r0 = __builtin_bit_cast(float, (uint32_t)r[0]), r1 = __builtin_bit_cast(float, (uint32_t)r[1]);
  return sum ? r0 + r1 : fmaxf(r0, r1);
}
__device__ __forceinline__ float wave_max_xor16_32(float v) { return xor16_32_pair_max(v, false); }
__device__ __forceinline__ float wave_sum_xor16_32(float v) { return xor16_32_pair_max(v, true); }

// Four OCP e4m3 codes (one dword) to four bf16 values, exactly (every e4m3 value is a
// bf16 value): the gfx950 scaled pair conversion with scale 1.
__device__ __forceinline__ uint2 e4m3x4_to_bf16x4(uint32_t w) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ uint16_t bf16_bits_rne(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

}  // namespace mla

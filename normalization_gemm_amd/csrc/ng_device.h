// Device-side helpers shared by the libnormgemm kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ng {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) float lds_float;
typedef __attribute__((address_space(3))) f32x2 lds_f32x2;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

// bf16 <-> fp32.  bf16 is the upper half of an fp32 bit pattern.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair (element 0 in the low half), round to nearest
// even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// D(16x16, fp32) += Aop(16x32) * Bop(32x16), bf16 operands.
// Lane l supplies Aop row (l % 16) and Bop column (l % 16), each with the 8
// k-values 8*(l/16) .. 8*(l/16)+7; D element (4*(l/16) + r, l % 16) lands in
// register r.  (Lane layout checked on the device against a host product.)
__device__ __forceinline__ f32x4 mfma_16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ lds_char* lds_base(void* smem) { return (lds_char*)smem; }

// 16-byte LDS access at a byte offset.
__device__ __forceinline__ u32x4 lds_read16(lds_char* base, uint32_t off) {
  return *(lds_u32x4*)(base + off);
}
__device__ __forceinline__ void lds_write16(lds_char* base, uint32_t off, u32x4 v) {
  *(lds_u32x4*)(base + off) = v;
}

// Transposing 8-byte LDS read (ds_read_b64_tr_b16).  Within each group of 16
// lanes, let lane j point at four consecutive 16-bit elements e = 0..3; lane i
// then receives, in slot q, element (i % 4) of lane (i / 4 + 4 * q).  (Mapping
// checked on the device.)
__device__ __forceinline__ u32x2 lds_read_tr16(lds_char* base, uint32_t off) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + off));
  return __builtin_bit_cast(u32x2, v);
}

// Agent-scope relaxed atomics: loads and stores bypass the per-XCD L2 so that
// values written by a workgroup on another XCD are observed.
__device__ __forceinline__ void store_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int load_agent(const int* p) {
  return __hip_atomic_load(const_cast<int*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(int* p, int v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int add_agent(int* p, int v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until every memory operation this wave issued has completed.
__device__ __forceinline__ void wait_all_mem() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Cache policy of the output stores: nontemporal (nt), for streamed results
// that the kernel never reads back.  (Measured on MI355X: the 16 MiB output
// of a 65536 x 512 x 128 GEMM + LayerNorm stores ~3.5 us sooner than with the
// default policy, 19.5 against 23.1 us per call.)
constexpr int kStoreNT = 2;

// Raw buffer resource over `bytes` bytes from `base`: loads at offsets at or
// beyond the size return zero.  Sizes are clamped below 2^31 so that offset
// kOOB is always out of range.
constexpr uint32_t kOOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0x7FFFFFF0ull ? 0x7FFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint32_t umin32(uint32_t a, uint32_t b) { return a < b ? a : b; }

// A value that is the same in every lane, kept in a scalar register (buffer
// resources must be built from scalar registers).
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

// The same with a size the caller has already brought to at most 0x7FFFFFF0.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const void* base, uint32_t n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)n, 0x00020000);
}

// 16 bytes per lane from global memory straight into LDS (buffer_load_dwordx4
// ... lds): lane l's data lands at LDS byte address lds_addr + 16*l; lds_addr
// must be wave-uniform.  Issued through inline asm so that the compiler does
// not add a full vmcnt wait before unrelated LDS reads; callers order the
// transfer with wait_vmcnt() and a barrier.  M0 is left holding the LDS
// address: nothing else in the library's kernels reads M0 (no s_movrel,
// s_sendmsg, GWS, ds_*_addtid or compiler-issued LDS transfers; a CPU test
// scans the compiled code for them), and saving and restoring it put two
// more scalar instructions beside every transfer of the k-loop (~0.7 % on
// the large shapes).
// NT: nontemporal load, for data that no other workgroup reads (a row block
// of A whose rows fit one column tile); data shared through L2 must not use
// it (measured ~10 % slower on the large shapes, whose A panels are re-read
// by every column tile).
template <bool NT = false>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t lds_addr, uint32_t voff,
                                      uint32_t soff) {
  if constexpr (NT) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
        :
        : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(lds_addr), "v"(voff), "s"(rs), "s"(soff)
        : "memory");
  }
}

// Wait until at most N vector-memory operations of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(lds_char* p) { return (uint32_t)(uintptr_t)p; }

}  // namespace ng

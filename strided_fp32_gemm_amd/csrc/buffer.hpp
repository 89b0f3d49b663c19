// buffer.hpp -- vector types and raw buffer-resource access for the gfx950
// kernels.
//
// Loads and stores go through buffer resources.  A lane outside its operand
// gets an offset beyond the resource's range, so the hardware returns zero
// for its load and drops its store: no branch and no access outside the
// operands.
#pragma once

#include <hip/hip_runtime.h>

namespace sgemm {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Raw buffer resources: stride 0, num_records = 2^31 bytes.  Offsets at or
// beyond kOutOfRange fail the hardware range check (loads read 0, stores are
// dropped).  Word 3 holds the gfx9-family data-format bits.
constexpr unsigned kOutOfRange = 0x80000000u;
constexpr int kRecordBytes = int(0x80000000u);
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const float *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, kRecordBytes, kRsrcWord3);
}

__device__ __forceinline__ f32x4 load4(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0));
}

__device__ __forceinline__ f32x2 load2(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(r, int(off), 0, 0));
}

__device__ __forceinline__ float load1(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, int(off), 0, 0));
}

__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, unsigned off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, v), r, int(off), 0, 0);
}

__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, int(off), 0, 0);
}

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedVmemRead = 0x020, kSchedVmemWrite = 0x040, kSchedLdsRead = 0x100,
              kSchedLdsWrite = 0x200;

// Device-scope store (cache-policy operand 16 sets sc1): the line goes out to
// the memory side of the fabric instead of collecting as a dirty line in the
// XCD's L2.  The short-k kernels, whose time is set by streaming their
// outputs, measured 4-5% faster with it; the LDS-tiled kernels measured up to
// 1% slower, so they keep the default policy.
constexpr int kStoreDevice = 16;

__device__ __forceinline__ void store4_device(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, int(off), 0, kStoreDevice);
}

}  // namespace sgemm

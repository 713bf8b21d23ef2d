// Memory-pipeline helpers shared by the kernels of libsa.so (gfx950): explicit vmcnt /
// lgkmcnt waits, a workgroup barrier that the compiler may not move memory accesses
// across, and 16-byte buffer loads that write LDS directly.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

// wait until at most N vector-memory operations of this wave are outstanding
template <int N>
static __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// wait for this wave's LDS and scalar-memory operations only
static __device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

static __device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef int v4i __attribute__((ext_vector_type(4)));

// buffer resource of `bytes` bytes at `base` (raw buffer, no stride)
static __device__ __forceinline__ v4i buffer_rsrc(const void* base, uint32_t bytes) {
    v4i r;
    r[0] = (int)(uint32_t)(uintptr_t)base;
    r[1] = (int)(uint32_t)((uintptr_t)base >> 32);
    r[2] = (int)bytes;
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from buffer offset voff + soff into LDS at lds + 16 * lane.  Written as asm so
// that the compiler does not order later LDS reads behind it: the kernel's own vmcnt waits
// and barriers order every read of the written data.  Offsets past the buffer's size move
// no data and write zeros.
static __device__ __forceinline__ void lds_dma16(const v4i& rs, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(__builtin_amdgcn_readfirstlane(lds)),
                 "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "m0");
}

// The same transfer from a full 64-bit address per lane (no buffer resource, so no 4 GiB
// window and no range check: every lane must point at readable memory).
static __device__ __forceinline__ void lds_dma16_g(uint32_t lds, const void* src) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(__builtin_amdgcn_readfirstlane(lds)), "v"(src)
                 : "m0");
}

// LDS byte address of a __shared__ object
static __device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

}  // namespace sa

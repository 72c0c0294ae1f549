// Buffer->LDS DMA and wait helpers for gfx950 (CDNA4): buffer resources over a
// byte range, wave-wide 16- and 4-byte global->LDS loads, and the waits and
// barrier that let such loads stay in flight across LDS reads of other buffers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmm {

#define QMM_G1 __attribute__((address_space(1)))
#define QMM_L3 __attribute__((address_space(3)))

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier for the LDS stages.  A release fence would wait for every
// outstanding global->LDS DMA (they count as LDS writes), including the prefetches
// that must stay in flight; instead each wave waits explicitly for the DMA it needs
// (wait_vm) and for its own LDS stores (lgkmcnt), and the empty asm statements keep
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0) only
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Buffer resource over [base, base + bytes) (raw addressing, 32-bit data format;
// reads past `bytes` return zeros instead of faulting).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = static_cast<int>(bytes < 0x7FFFFFFF ? bytes : 0x7FFFFFFF);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

// Cache policy of a DMA load: kCacheNT marks data that is read once (streamed
// weights), so it does not displace reused data in the caches.
constexpr int kCacheDefault = 0;
constexpr int kCacheNT = 2;

// One 16-byte buffer->LDS DMA per lane: lane L's bytes (resource + voff + soff) land
// at lds + 16 L.
template <int POL = kCacheDefault>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, QMM_L3 uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (QMM_L3 void*)lds, 16, static_cast<int>(voff), static_cast<int>(soff), 0,
                                             POL);
}

// One 4-byte buffer->LDS DMA per lane: lane L's dword (resource + voff) lands at
// lds + 4 L.
template <int POL = kCacheDefault>
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint32_t voff, QMM_L3 uint8_t* lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (QMM_L3 void*)lds, 4, static_cast<int>(voff), 0, 0, POL);
}

}  // namespace qmm

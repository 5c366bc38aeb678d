// Direct-to-LDS tile loading for the gfx950 matrix-core kernels (the map GEMM and the fit
// side's co-moment GEMM): buffer descriptors, buffer_load_dwordx4 ... lds, the row swizzle
// of 128-byte tile rows, explicit vmcnt waits and a branch-free uniform select.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace kvmap {
namespace {

// LDS slot of the 16-byte chunk c (0..7) of tile row r is c ^ slot_xor(r).  Rows are 128
// bytes.  For the rows r..r+15 read by 16 consecutive lanes of a ds_read_b128 (one chunk
// index), (r & 1, c ^ slot_xor(r)) covers all 16 bank groups of a 256-byte (64-bank)
// window, and for 8 consecutive lanes c ^ slot_xor(r) covers the 8 groups of a 128-byte
// window: conflict free under either bank count.
__device__ __forceinline__ int slot_xor(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Buffer descriptor over [base, base + bytes) for raw buffer loads (gfx9 dword3 = 0x00020000).
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    const i32x4_t r = {__builtin_amdgcn_readfirstlane((int)(uint32_t)b),
                       __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32)), (int)bytes, 0x00020000};
    return r;
}

// buffer_load_dwordx4 ... lds: 16 bytes per lane from rsrc + voff + soff into LDS at
// m0 + 16 * lane.  Written as inline assembly so that the compiler's conservative waits
// for direct-to-LDS loads (it cannot tell the pipeline's stage buffers apart and would
// drain every load before issuing the next stage) stay out of the pipeline; the kernel
// orders these loads itself with explicit vmcnt waits and barriers.  Nothing else in the
// kernel uses m0.
__device__ __forceinline__ void lds_dma16(i32x4_t rsrc, uint32_t lds_addr, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// The same load with the non-temporal hint: for data read exactly once (a stream of map
// weights), so that it does not displace lines that other workgroups will read again.
__device__ __forceinline__ void lds_dma16_nt(i32x4_t rsrc, uint32_t lds_addr, int voff, int soff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}

// One dword at a wave-uniform address through the scalar cache (a read; the wait for it is
// part of the statement, so the result is ready when it ends).  For small tables read inside
// a pipeline whose vector-memory counter must only count the pipeline's own loads.
__device__ __forceinline__ int scalar_load_dword(const int32_t* p) {
    int r;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=&s"(r) : "s"(p) : "memory");
    return r;
}

// c ? a : b on uniform values, as one s_cselect.  Written out because the compiler turns a
// select between a v_readlane result and an add into a branch, which would split the loop.
__device__ __forceinline__ uint32_t uniform_select(uint32_t c, uint32_t a, uint32_t b) {
    uint32_t r;
    asm("s_cmp_lg_u32 %1, 0\n\ts_cselect_b32 %0, %2, %3"
        : "=s"(r)
        : "s"(__builtin_amdgcn_readfirstlane(c)), "s"(a), "s"(b)
        : "scc");
    return r;
}

// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace
}  // namespace kvmap

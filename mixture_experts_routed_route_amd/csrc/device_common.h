// Device helpers shared by the gfx950 kernels of the MoE expert path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t h) {
    return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 -> packed pair of bf16 (low half = a), one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// SiLU(g) * u with a hardware reciprocal (1 ulp) instead of an IEEE division.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// Inclusive prefix sum of `v` over the 64 lanes of a wave with DPP: shifts by 1, 2, 4 and 8
// lanes inside each row of 16, then row 0's and row 2's last lane into the rows after them
// (row_bcast:15) and lane 31 into rows 2 and 3 (row_bcast:31).  Lanes without a source add 0.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15, rows 1 and 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31, rows 2 and 3
    return v;
}

// Inclusive prefix sum of `v` over the first `active` waves of a block of NW waves (values of
// later waves are ignored); the result is defined on those waves only.  `scratch` holds >= NW
// ints.  Every thread of the block must call it with the same `active`.  With one active wave
// there is no exchange and no barrier; otherwise the barriers order LDS only.
template <int NW>
__device__ __forceinline__ int block_inclusive_scan(int v, int* scratch, int active = NW) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    v = wave_inclusive_scan(v);
    if (active <= 1) return v;
    if (lane == 63) scratch[wave] = v;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    int add = 0;
    const int nw = wave < active ? wave : 0;
    for (int w = 0; w < nw; ++w) add += scratch[w];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    return v + add;
}

__device__ __forceinline__ int block_inclusive_scan_256(int v, int* scratch) {
    return block_inclusive_scan<4>(v, scratch);
}

// Largest e in [0, n) with off[e] <= r (off non-decreasing, off[0] <= r).
__device__ __forceinline__ int upper_index(const int* off, int n, int r) {
    int lo = 0, hi = n;  // invariant: off[lo] <= r, answer in [lo, hi)
    while (hi - lo > 1) {
        int mid = (lo + hi) >> 1;
        if (off[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

// ------------------------------------------------------------------ direct global -> LDS loads
// A 16-byte chunk of zeros in device memory: the source of the lanes whose chunk lies past a range.
__device__ __attribute__((aligned(16))) const uint32_t kZero16[4] = {0u, 0u, 0u, 0u};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// 16 bytes per lane from global memory straight into LDS at m0 + lane*16 (one 1 KB row block
// per wave).  Emitted as inline asm so that the compiler does not treat every later LDS read
// as dependent on it (it would drain all loads in flight before each read); completion is
// tracked with explicit vmcnt waits instead.  m0 is written inside the statement itself.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds_addr) : "memory");
}

// The same with the source as a scalar base plus a 32-bit per-lane byte offset (saddr form).
__device__ __forceinline__ void dma16_s(const void* base, uint32_t off, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(lds_addr)
                 : "memory");
}

// 4 bytes per lane from global memory straight into LDS at m0 + lane*4 (256 bytes per wave), for
// small staging that the compiler must not track (see dma16).
__device__ __forceinline__ void dma4(const void* g, uint32_t lds_addr) {
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr) : "memory");
}

// A wave-uniform pointer held in scalar registers (a select between two uniform pointers may
// otherwise be formed in vector registers, which an "s" operand cannot take).
template <typename T>
__device__ __forceinline__ const T* uniform_ptr(const T* p) {
    const uint64_t v = reinterpret_cast<uintptr_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
    return reinterpret_cast<const T*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// LDS byte address of a __shared__ object (wave-uniform)
__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(p))));
}

}  // namespace moe

// Device helpers shared by the HIP kernel files (dgrad_kernels.hip,
// dgrad_wide.hip, chain_kernels.hip): vector types, raw buffer resources with
// the hardware range check, the direct-to-LDS 16-byte load, the LDS chunk
// permutations, the activation derivative g(z) of the fused epilogue, and the
// workgroup -> XCD placement. Not part of the public ABI.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace cbw {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Buffer resources for raw, unswizzled 32-bit-format buffer accesses. A lane
// whose offset is at or past the buffer size reads zeros and has its store
// dropped by the hardware range check; 2^31 is such an offset for every
// tensor the host admits (all are below 2^31 bytes).
constexpr int kRawBufferFlags = 0x00020000;

// Cache policies of output stores (an output is written once and never read
// back by the kernel). kStoreNT, the non-temporal hint, keeps its lines from
// displacing operand lines in L2. kStoreSystem, sc0 sc1 (system scope), sends
// them on towards memory instead of leaving them dirty in L2; it is the
// better one where most of a launch's bytes are stores, as in layers whose
// zero phases are stored beside the GEMM pixels. Measured on MI355X, cold: the
// 1x1 stride-2 layer (617 MB, two-thirds stores) 145-149 us with kStoreSystem
// against 168-171 us with kStoreNT; elsewhere kStoreNT is equal or better
// (the fused two-step chain 180-198 against 205-216 us, the forward 1x1
// stride-2 layer 155-159 against 171-172 us).
constexpr int kStoreNT = 2;
constexpr int kStoreSystem = 17;

// Byte offset for a buffer access: `off` itself (below 2^31 for an in-range
// lane), or exactly 2^31 when bad == 1. Arithmetic, not a select, so no branch
// is formed around the access. A caller may add up to 2^31 - 1 more bytes to
// a bad offset and still stay out of range without wrapping.
__device__ inline uint32_t out_of_range_if(uint32_t bad, uint32_t off)
{
    return (off & (bad - 1u)) | (bad << 31);
}

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kRawBufferFlags);
}

// The same descriptor as four dwords (base, stride 0, size, format), for the
// inline-assembly loads.
__device__ inline i32x4 raw_descriptor(const void* base, uint32_t bytes)
{
    const uint64_t p = (uint64_t)base;
    return i32x4{(int)(uint32_t)p, (int)((p >> 32) & 0xffffu), (int)bytes, kRawBufferFlags};
}

// One 16-byte direct-to-LDS load per lane: LDS[lds_base + 16*lane] <-
// buffer[voffset + soffset] (soffset wave-uniform). An in-range lane has
// voffset + soffset inside the buffer; an out-of-range lane has voffset =
// 2^31 (and soffset < 2^31), outside the buffer however the hardware combines
// the two offsets for its range check. The load writes LDS, not registers,
// so the asm has no output operand; its completion is awaited with vmcnt.
__device__ inline void dma16(i32x4 desc, uint32_t voffset, uint32_t soffset, uint32_t lds_base)
{
    const int so = __builtin_amdgcn_readfirstlane((int)soffset);   // uniform by construction
    const int lb = __builtin_amdgcn_readfirstlane((int)lds_base);
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(desc), "s"(so), "s"(lb)
                 : "memory", "m0");
}

// The same load with the LDS address formed in m0 from a wave-uniform base
// plus a compile-time byte offset: one scalar add per load (it sets SCC,
// hence the clobber).
template <uint32_t OFF>
__device__ inline void dma16_at(i32x4 desc, uint32_t voffset, uint32_t soffset, uint32_t lds_base)
{
    // every scalar operand taken from the first lane (uniform by construction),
    // so the compiler holds it in scalar registers whatever it can prove
    const i32x4 d{__builtin_amdgcn_readfirstlane(desc.x), __builtin_amdgcn_readfirstlane(desc.y),
                  __builtin_amdgcn_readfirstlane(desc.z), __builtin_amdgcn_readfirstlane(desc.w)};
    const int so = __builtin_amdgcn_readfirstlane((int)soffset);
    const int lb = __builtin_amdgcn_readfirstlane((int)lds_base);
    asm volatile("s_add_u32 m0, %3, %4\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
                 :
                 : "v"(voffset), "s"(d), "s"(so), "s"(lb), "n"(OFF)
                 : "memory", "m0", "scc");
}

// Compile-time integers as values (IC<N>{}), and a loop over them whose body
// sees its index as a constant expression (decltype(i)::value).
template <int N>
struct IC {
    static constexpr int value = N;
};

template <int B, int E, typename F>
__device__ inline void static_for(F&& f)
{
    if constexpr (B < E) {
        f(IC<B>{});
        static_for<B + 1, E>(f);
    }
}

// A wave-uniform 32-bit value kept in a scalar register: the compiler may
// not re-derive it later from the kernel arguments (a scalar memory load,
// whose wait would also drain the LDS reads in flight). The value is taken
// from the first active lane, which is exact for a uniform value wherever the
// compiler happened to hold it.
template <typename T>
__device__ inline T pin(T x)
{
    static_assert(sizeof(T) == 4, "32-bit values");
    int v = __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x));
    asm volatile("" : "+s"(v));
    return __builtin_bit_cast(T, v);
}

template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Chunk (16-byte) permutation of pixel rows in LDS (128-byte rows): chunk c of
// row m sits at position c ^ ((m >> 1) & 7), so 16 lanes reading one chunk of
// 16 consecutive rows hit 16 distinct 16-byte bank groups of the 256-byte
// bank window.
__device__ inline int dy_swizzle(int row)
{
    return (row >> 1) & 7;
}

// Chunk permutation of filter row k in LDS (rows of B_ROW bytes). A
// transpose read covers, per 32-lane half, four consecutive rows x four
// consecutive chunks; the permutation sends these 16 (row, chunk) pairs to
// 16 distinct 16-byte bank groups of the 256-byte bank window.
template <int B_ROW>
__device__ inline int w_swizzle(int k)
{
    static_assert(B_ROW == 128 || B_ROW % 256 == 0, "filter rows of 128 bytes or whole bank windows");
    return B_ROW == 128 ? 4 * ((k >> 1) & 1) : 4 * (k & 3);
}

constexpr int kEpiNone = 0;
constexpr int kEpiDRelu = 1;
constexpr int kEpiDHardswish = 2;

// g(z) for the fused epilogues, evaluated in fp32 without branches, for z
// converted from fp16 (every caller's z is an fp16 tensor).
// g = 1 (none); relu'(z) = [z > 0]; hardswish'(z) = 0 below -3, z/3 + 1/2 on
// the closed interval [-3, 3], 1 above 3, where z/3 is the correctly rounded
// fp32 quotient. It is formed without a division: q0 = z * RN(1/3), the
// residual z - 3*q0 (exact in one fused multiply-add), then q0 plus the
// residual times RN(1/3). For every fp16 z in [-3, 3] this equals the
// correctly rounded quotient (checked exhaustively on the host); the
// division sequence it replaces cost about a dozen instructions per value.
constexpr float kThirdRN = 0x1.555556p-2f;   // RN(1/3) in fp32

template <int E>
__device__ inline float epilogue_factor(float z)
{
    if constexpr (E == kEpiNone)
        return 1.0f;
    if constexpr (E == kEpiDRelu)
        return z > 0.0f ? 1.0f : 0.0f;
    const float q0 = z * kThirdRN;
    const float q = __builtin_fmaf(__builtin_fmaf(-3.0f, q0, z), kThirdRN, q0);
    const float mid = q + 0.5f;
    return z < -3.0f ? 0.0f : (z > 3.0f ? 1.0f : mid);
}

template <int E>
struct EpiTag {
    static constexpr int value = E;
};

// Hardware dispatch places workgroup b on XCD (b mod 8) as that XCD's
// (b div 8)-th workgroup; each XCD has its own L2. Two placements of logical
// tiles [0, total) (both bijections):
//   mode 0: each XCD gets whole groups of `g` consecutive logical tiles
//           (tiles that share operands, e.g. the channel tiles of one pixel
//           block), groups rotating over the XCDs so a heavy-first phase
//           order stays balanced; a tail that fills no 8 groups goes to
//           the XCDs in contiguous ranges, as in mode 1, so that a group of
//           the tail shares fewer L2s (two, for 32 tail workgroups in
//           groups of 8, where round-robin placement gave eight).
//   mode 1: each XCD gets one contiguous eighth of the logical tiles (tiles
//           ordered so that neighbours share operands then share an L2).
__device__ inline int xcd_remap(int b, int total, int g, int mode)
{
    const int x = b & 7;
    const int l = b >> 3;
    if (mode == 1) {
        const int q = total >> 3, r = total & 7;
        return x * q + (x < r ? x : r) + l;
    }
    const int span = 8 * g;
    const int main_part = (total / span) * span;
    if (b >= main_part) {        // main_part is a multiple of 8: b and b - main_part share the XCD
        const int t = b - main_part, rest = total - main_part;
        const int xt = t & 7, lt = t >> 3;
        const int q = rest >> 3, r = rest & 7;
        return main_part + xt * q + (xt < r ? xt : r) + lt;
    }
    return ((l / g) * 8 + x) * g + (l % g);
}

}  // namespace cbw

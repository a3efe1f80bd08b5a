// Device helpers shared by the two decode attention kernels (bf16 cache and
// FP8 cache): scalar table reads, the VGPR-form score MFMAs, LDS operand reads
// and the HBM -> LDS tile copy.
#pragma once

#include "device_util.h"

namespace mla {
namespace attn {

#define MLA_CONST __attribute__((address_space(4)))
// Read-only tables go through the constant address space so that wave-uniform
// lookups become scalar loads (counted by lgkmcnt, never waiting on the
// in-flight tile copies, which are counted by vmcnt).
template <typename T>
__device__ __forceinline__ const MLA_CONST T* as_const(const T* p) {
  return (const MLA_CONST T*)p;
}

__device__ __forceinline__ bf16x8 as_bf8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Score MFMAs with their accumulators in VGPRs (the latent accumulators fill the
// AGPRs).  Written as asm so that the choice is per instruction; the hazards
// the compiler would otherwise handle are handled here: a chain starts from a
// literal zero (no vector write precedes it), a chain accumulates in place with
// the same opcode (back-to-back dependent issue is supported), and the results
// are read only after settle's wait states.
__device__ __forceinline__ void mfma_s_first(f32x16& acc, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16& acc, u32x4 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// 24 wait states: more than an 8- or 16-pass MFMA's result needs before a vector read
__device__ __forceinline__ void settle_s(f32x16& a0) { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0)); }
__device__ __forceinline__ void settle_s(f32x16& a0, f32x16& a1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}
__device__ __forceinline__ void settle_s(f32x16& a0, f32x16& a1, f32x16& a2) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1), "+v"(a2));
}

__device__ __forceinline__ u32x4 lds_read16(const MLA_LDS uint8_t* p) { return *(const MLA_LDS u32x4*)p; }

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4 e + q points at 4 bf16 of row e
// (e = 0..3); lane i of the group receives element i of the 16-wide block of each row
__device__ __forceinline__ u32x2 lds_read_tr16(const MLA_LDS uint8_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((MLA_LDS s16x4*)p);
  return __builtin_bit_cast(u32x2, v);
}

// One 16-byte-per-lane copy HBM -> LDS: global address = base + voff, LDS
// address = m0 + 16 * lane.  Issued as asm so that the compiler does not
// treat every later LDS read as aliasing the copy (it would then wait for all
// copies in flight); the ring protocol waits for exactly the stage it reads.
// The cache stream is read once, so it is marked non-temporal: it then
// displaces less of what the step's other kernels re-read from the caches.
__device__ __forceinline__ void copy16_to_lds(uint64_t base, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base), "s"(lds_addr)
               : "memory");
}

// a wave-uniform 64-bit address, made visibly uniform (scalar registers)
__device__ __forceinline__ uint64_t uniform_addr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}


// ---- Partial latent sums out of the accumulators: rounded to bf16, row-major [row][512].
// The 128 rows go through LDS in passes of 32: the kernel writes a pass's fp32
// accumulators to LDS straight from the AGPRs (stage_row_f4), then every thread
// converts a few values at a time and stores whole 128-byte runs (store_pass_bf16).
// Converting in registers instead would move all 256 accumulators into VGPRs at
// once, which costs the main loop its registers.
constexpr int kEpiRows = 32;
constexpr int kEpiStride = kLat * 4 + 16;   // padded fp32 row in LDS
static_assert(kEpiRows * kEpiStride <= 120 * 1024, "an epilogue pass fits the ring");

// fp32 x4 of row r (0..31 within the pass), features f .. f + 3
__device__ __forceinline__ void stage_row_f4(MLA_LDS uint8_t* lds, int r, int f, f32x4 v) {
  *(MLA_LDS f32x4*)(lds + r * kEpiStride + f * 4) = v;
}
// 256 threads: the pass's 32 rows to out_rows[r * kLat ..] (bf16); row r is written only if
// r < nrows
__device__ __forceinline__ void store_pass_bf16(const MLA_LDS uint8_t* lds, uint16_t* out_rows, int tid) {
  const int r = tid >> 3, part = tid & 7;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int f = 8 * (8 * j + part);
    const f32x4 a = *(const MLA_LDS f32x4*)(lds + r * kEpiStride + f * 4);
    const f32x4 b = *(const MLA_LDS f32x4*)(lds + r * kEpiStride + f * 4 + 16);
    *(u32x4*)(out_rows + (size_t)r * kLat + f) =
        u32x4{pack_bf2(a[0], a[1]), pack_bf2(a[2], a[3]), pack_bf2(b[0], b[1]), pack_bf2(b[2], b[3])};
  }
}

}  // namespace attn
}  // namespace mla
